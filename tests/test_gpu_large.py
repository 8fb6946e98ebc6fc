"""Tensors of more than 2^31 elements (64-bit indexing), one per operator.

Inputs are drawn on the GPU from torch's seeded generator (host generation of
~4 GB per tensor would dominate the run); the oracle then checks sampled rows
or images on both sides of the 2^31-element boundary, copied to the host.
Each test holds 13-17 GB of device memory and frees it before the next."""
import gc

import numpy as np
import pytest
import torch

import group_normalization_amd as gn
import oracle
from parity import assert_bitwise, assert_close

pytestmark = pytest.mark.gpu

TWO31 = 2 ** 31


def gen(shape, dtype, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return torch.randn(shape, dtype=torch.float32, device="cuda", generator=g).to(dtype)


@pytest.fixture(autouse=True)
def free_memory():
    yield
    gc.collect()
    torch.cuda.empty_cache()


def test_ssln_beyond_2_31_elements():
    hidden = 4096
    rows = TWO31 // hidden + 8
    x = gen((rows, hidden), torch.float16, 1)
    k = gen((rows, hidden), torch.float16, 2)
    gamma = (torch.rand(hidden, device="cuda", generator=torch.Generator(device="cuda").manual_seed(3)) + 0.5).half()
    out = gn.skip_rms_norm(x, k, gamma, None, 1e-6, want_inv_std_var=True, want_sum=True)
    assert gn.last_route() == "ssln.wave2.vec16"
    torch.cuda.synchronize()
    sample = np.array([0, 1, TWO31 // hidden - 1, TWO31 // hidden, rows - 2, rows - 1])
    idx = torch.from_numpy(sample).cuda()
    xs, ks = x[idx].cpu().numpy(), k[idx].cpu().numpy()
    ref = oracle.skip_rms_norm(xs, ks, gamma.cpu().numpy(), None, 1e-6, want_inv_std_var=True,
                               want_sum=True)
    assert_close(out.output[idx].cpu().numpy(), ref[0], "output")
    assert_close(out.inv_std_var[idx].cpu().numpy(), ref[2], "inv_std_var")
    assert_bitwise(out.input_skip_bias_sum[idx].cpu().numpy(), ref[3], "S")


def test_gated_beyond_2_31_elements():
    C = 128
    rows = TWO31 // C + 64
    X = gen((rows, C), torch.float16, 4)
    G = gen((rows, C), torch.float16, 5)
    scale = (torch.rand(C, device="cuda", generator=torch.Generator(device="cuda").manual_seed(6)) + 0.5).half()
    Y = gn.gated_rms_norm(X, scale, G, 1e-5)
    assert gn.last_route() == "gated.segment.vec16"
    torch.cuda.synchronize()
    sample = np.array([0, TWO31 // C - 1, TWO31 // C, rows - 1])
    idx = torch.from_numpy(sample).cuda()
    ref = oracle.gated_rms_norm(X[idx].cpu().numpy(), scale.cpu().numpy(), G[idx].cpu().numpy(), 1e-5)
    assert_close(Y[idx].cpu().numpy(), ref, "Y")


def test_skip_layer_norm_beyond_2_31_elements():
    hidden = 4096
    rows = TWO31 // hidden + 8
    x = gen((rows, hidden), torch.float16, 11)
    k = gen((rows, hidden), torch.float16, 12)
    g = torch.Generator(device="cuda").manual_seed(13)
    gamma = (torch.rand(hidden, device="cuda", generator=g) + 0.5).half()
    beta = (0.1 * torch.randn(hidden, device="cuda", generator=g)).half()
    out = gn.skip_layer_norm(x, k, gamma, beta, None, 1e-5, want_mean=True, want_sum=True)
    assert gn.last_route() == "ssln.wave2.vec16"
    torch.cuda.synchronize()
    sample = np.array([0, TWO31 // hidden - 1, TWO31 // hidden, rows - 1])
    idx = torch.from_numpy(sample).cuda()
    ref = oracle.skip_layer_norm(x[idx].cpu().numpy(), k[idx].cpu().numpy(), gamma.cpu().numpy(),
                                 beta.cpu().numpy(), None, 1e-5, want_mean=True, want_sum=True)
    assert_close(out.output[idx].cpu().numpy(), ref[0], "output")
    assert_close(out.mean[idx].cpu().numpy(), ref[1], "mean")
    assert_bitwise(out.input_skip_bias_sum[idx].cpu().numpy(), ref[3], "S")


@pytest.mark.parametrize("C,route", [(16384, "gated.row.vec16"), (132, "gated.flat.vec16"),
                                     (301, "gated.flat.vec16")])
def test_gated_wide_and_flat_rows_beyond_2_31_elements(C, route):
    rows = TWO31 // C + 64
    X = gen((rows, C), torch.float16, 14)
    G = gen((rows, C), torch.float16, 15)
    scale = (torch.rand(C, device="cuda", generator=torch.Generator(device="cuda").manual_seed(16)) + 0.5).half()
    Y = gn.gated_rms_norm(X, scale, G, 1e-5)
    assert gn.last_route() == route
    torch.cuda.synchronize()
    sample = np.array([0, TWO31 // C - 1, TWO31 // C, TWO31 // C + 1, rows - 1])
    idx = torch.from_numpy(sample).cuda()
    ref = oracle.gated_rms_norm(X[idx].cpu().numpy(), scale.cpu().numpy(), G[idx].cpu().numpy(), 1e-5)
    assert_close(Y[idx].cpu().numpy(), ref, "Y")


@pytest.mark.parametrize("channels_last", [1, 0])
def test_sgn_beyond_2_31_elements(channels_last):
    C, H, W, groups = 256, 16, 16, 32
    per_image = C * H * W
    N = TWO31 // per_image + 1
    shape = (N, H, W, C) if channels_last else (N, C, H, W)
    X = gen(shape, torch.float16, 7)
    skip = gen(shape, torch.float16, 8)
    rng = np.random.default_rng(9)
    gamma = torch.from_numpy(rng.uniform(0.5, 1.5, C).astype(np.float32)).cuda()
    beta = torch.from_numpy((0.1 * rng.standard_normal(C)).astype(np.float32)).cuda()
    bias = torch.from_numpy((0.1 * rng.standard_normal(C)).astype(np.float16)).cuda()
    out = gn.skip_group_norm(X, gamma, beta, skip, bias, groups=groups, activation=1,
                             channels_last=channels_last, want_sum=True)
    torch.cuda.synchronize()
    for n in (0, TWO31 // per_image - 1, N - 1):
        ref_y, ref_s = oracle.skip_group_norm(X[n:n + 1].cpu().numpy(), gamma.cpu().numpy(),
                                              beta.cpu().numpy(), skip[n:n + 1].cpu().numpy(),
                                              bias.cpu().numpy(), groups=groups, activation=1,
                                              channels_last=channels_last, want_sum=True)
        assert_close(out.Y[n:n + 1].cpu().numpy(), ref_y, f"Y image {n}")
        assert_bitwise(out.S[n:n + 1].cpu().numpy(), ref_s, f"S image {n}")


def test_sgn_packed_runs_beyond_2_31_elements():
    """NHWC pixels of 15 float16 channels (runs of 8 pixels make 15 whole
    16-byte vectors): the cluster over packed runs, in many rounds of
    resident workgroups, past the 2^31-element boundary."""
    C, H, W, groups = 15, 264, 264, 5
    per_image = C * H * W
    N = TWO31 // per_image + 2
    X = gen((N, H, W, C), torch.float16, 17)
    skip = gen((N, H, W, C), torch.float16, 18)
    rng = np.random.default_rng(19)
    gamma = torch.from_numpy(rng.uniform(0.5, 1.5, C).astype(np.float32)).cuda()
    beta = torch.from_numpy((0.1 * rng.standard_normal(C)).astype(np.float32)).cuda()
    bias = torch.from_numpy((0.1 * rng.standard_normal(C)).astype(np.float16)).cuda()
    out = gn.skip_group_norm(X, gamma, beta, skip, bias, groups=groups, activation=1, channels_last=1,
                             want_sum=True)
    assert "packed" in gn.last_route(), gn.last_route()
    torch.cuda.synchronize()
    for n in (0, TWO31 // per_image, N - 1):  # the middle one straddles element 2^31
        ref_y, ref_s = oracle.skip_group_norm(X[n:n + 1].cpu().numpy(), gamma.cpu().numpy(),
                                              beta.cpu().numpy(), skip[n:n + 1].cpu().numpy(),
                                              bias.cpu().numpy(), groups=groups, activation=1,
                                              channels_last=1, want_sum=True)
        assert_close(out.Y[n:n + 1].cpu().numpy(), ref_y, f"Y image {n}")
        assert_bitwise(out.S[n:n + 1].cpu().numpy(), ref_s, f"S image {n}")
