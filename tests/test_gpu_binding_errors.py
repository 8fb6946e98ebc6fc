"""Contract violations reach the caller from the C library's own validation:
the binding passes every tensor as a descriptor and checks nothing itself, so
each case below is rejected in C (before anything is enqueued) and surfaces
as SkipNormError with the library's status and message."""
import pytest
import torch

import group_normalization_amd as gn
from group_normalization_amd import SkipNormError

pytestmark = pytest.mark.gpu


def t(*shape, dtype=torch.float16):
    return torch.zeros(shape, dtype=dtype, device="cuda")


def expect(status, text, fn, *args, **kw):
    with pytest.raises(SkipNormError) as e:
        fn(*args, **kw)
    assert e.value.status_name == status and text in str(e.value), str(e.value)


def test_ssln_contract():
    x = t(4, 64)
    expect("SN_ERR_SHAPE", "input must have rank 2", gn.skip_rms_norm, t(256), t(256), t(64))
    expect("SN_ERR_SHAPE", "skip must have shape (4, 64)", gn.skip_rms_norm, x, t(4, 32), t(64))
    expect("SN_ERR_SHAPE", "gamma must have shape (64,)", gn.skip_rms_norm, x, t(4, 64), t(32))
    expect("SN_ERR_SHAPE", "bias must have shape (64,)", gn.skip_rms_norm, x, t(4, 64), t(64), t(1, 64))
    expect("SN_ERR_DTYPE", "skip must be float16", gn.skip_rms_norm, x, t(4, 64, dtype=torch.float32), t(64))
    expect("SN_ERR_DTYPE", "bfloat16", gn.skip_rms_norm, t(4, 64, dtype=torch.bfloat16),
           t(4, 64, dtype=torch.bfloat16), t(64, dtype=torch.bfloat16))
    expect("SN_ERR_ATTR", "epsilon", gn.skip_rms_norm, x, t(4, 64), t(64), None, -1.0)
    expect("SN_ERR_SHAPE", "beta must have shape (64,)", gn.skip_layer_norm, x, t(4, 64), t(64), t(63))


def test_gated_contract():
    x = t(8, 256)
    expect("SN_ERR_SHAPE", "scale must be a vector", gn.gated_rms_norm, x, t(2, 64), x.clone())
    expect("SN_ERR_SHAPE", "not a multiple of the span", gn.gated_rms_norm, x, t(100), x.clone())
    expect("SN_ERR_SHAPE", "gate must have shape (8, 256)", gn.gated_rms_norm, x, t(128), t(256, 8))
    expect("SN_ERR_DTYPE", "scale must be float16", gn.gated_rms_norm, x, t(128, dtype=torch.float32),
           x.clone())


def test_sgn_contract():
    X = t(2, 8, 8, 64)  # NHWC
    g, b = t(64, dtype=torch.float32), t(64, dtype=torch.float32)
    kw = dict(groups=8, activation=0)
    expect("SN_ERR_SHAPE", "X must have rank 4", gn.skip_group_norm, t(2, 64, 64), g, b, t(2, 64, 64), **kw)
    expect("SN_ERR_SHAPE", "skip must have X's shape", gn.skip_group_norm, X, g, b, t(2, 64, 1, 1), **kw)
    expect("SN_ERR_SHAPE", "skip must have X's shape", gn.skip_group_norm, X, g, b, t(1, 64), **kw)
    expect("SN_ERR_SHAPE", "gamma must have shape (64,)", gn.skip_group_norm, X, t(32, dtype=torch.float32),
           b, X.clone(), **kw)
    expect("SN_ERR_DTYPE", "beta must be float32", gn.skip_group_norm, X, g, t(64), X.clone(), **kw)
    expect("SN_ERR_SHAPE", "bias must have shape (64,)", gn.skip_group_norm, X, g, b, X.clone(), t(8), **kw)
    expect("SN_ERR_ATTR", "divide C", gn.skip_group_norm, X, g, b, X.clone(), groups=7, activation=0)
    expect("SN_ERR_ATTR", "activation", gn.skip_group_norm, X, g, b, X.clone(), groups=8, activation=2)
    # NCHW reads C from axis 1: the same tensor with 8 channels and groups 16.
    expect("SN_ERR_ATTR", "divide C", gn.skip_group_norm, X, t(8, dtype=torch.float32),
           t(8, dtype=torch.float32), X.clone(), groups=16, activation=0, channels_last=0)
    Y = torch.empty_like(X)
    expect("SN_ERR_SHAPE", "Y must have shape", gn.skip_group_norm_noalloc, X, g, b, X.clone(), groups=8,
           activation=0, Y=t(2, 64, 8, 8))
    # Both broadcast spellings are accepted.
    for skip in (t(2, 64), t(2, 1, 1, 64)):
        out = gn.skip_group_norm(X, g, b, skip, **kw)
        gn.skip_group_norm_noalloc(X, g, b, skip, Y=Y, **kw)
        torch.cuda.synchronize()
        assert torch.equal(out.Y, Y)
