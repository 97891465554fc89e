"""Host-side checks of the PyTorch layers: activation-name parsing, module
state compatible with torch.nn, and loud failure off the GPU (no fallback)."""
import pytest
import torch

import normalization_ln_rmsnorm_amd as nm


@pytest.mark.parametrize("name,expect", [
    (None, ("none", 0.0)), ("relu", ("relu", 0.0)), ("GELU", ("gelu", 0.0)),
    ("leaky_relu", ("leaky_relu", 0.01)), ("leaky_relu_0.2", ("leaky_relu", 0.2)),
    ("elu", ("elu", 1.0)), ("elu_0.5", ("elu", 0.5)), ("celu_2", ("celu", 2.0)),
    ("hardswish", ("hardswish", 0.0)), ("silu", ("silu", 0.0))])
def test_parse_act(name, expect):
    assert nm.parse_act(name) == expect


@pytest.mark.parametrize("bad", ["swish", "relu_0.5", "leaky_relu_x", "celu_0", "elu_nan", 3])
def test_parse_act_rejects(bad):
    with pytest.raises((ValueError, TypeError)):
        nm.parse_act(bad)


def test_state_dicts_match_torch():
    pairs = [(nm.LayerNorm(32), torch.nn.LayerNorm(32)),
             (nm.RMSNorm(32), torch.nn.RMSNorm(32)),
             (nm.BatchNorm1d(8, act_func="relu"), torch.nn.BatchNorm1d(8)),
             (nm.BatchNorm2d(8, act_func="gelu"), torch.nn.BatchNorm2d(8))]
    for ours, ref in pairs:
        assert isinstance(ours, type(ref))
        assert ours.state_dict().keys() == ref.state_dict().keys()
        ours.load_state_dict(ref.state_dict())


def test_cpu_tensors_fail_loudly():
    x = torch.randn(4, 32)
    with pytest.raises(ValueError, match="GPU"):
        nm.LayerNorm(32)(x)
    with pytest.raises(ValueError, match="GPU"):
        nm.RMSNorm(32)(x)
    with pytest.raises(ValueError, match="GPU"):
        nm.BatchNorm1d(32)(x)


def test_shape_checks():
    with pytest.raises(ValueError):
        nm.LayerNorm(16)(torch.randn(4, 32))
    with pytest.raises(ValueError):
        nm.BatchNorm2d(8)(torch.randn(2, 8, 3, 3), pre_act_add=torch.randn(2, 8, 3, 4))


def test_output_dtype_policy():
    bf = torch.bfloat16
    assert nm.output_dtype(bf, True) == torch.float32
    assert nm.output_dtype(bf, True, autocast_to_fp32=False) == bf
    assert nm.output_dtype(bf, False) == bf
    assert nm.output_dtype(bf, True, kind="batch_norm") == bf


def test_act_dropout_module_checks():
    with pytest.raises(ValueError):
        nm.ActDropout("gelu", drop_p=1.5)
    with pytest.raises(ValueError):
        nm.ActDropout("nope", drop_p=0.1)
    with pytest.raises(ValueError, match="GPU"):
        nm.ActDropout("gelu", drop_p=0.1)(torch.randn(8))
