"""C ABI behaviour that needs a GPU: a call's status reflects its own
launches only."""
import ctypes

import pytest
import torch

pytestmark = pytest.mark.gpu

nl = pytest.importorskip("normalization_ln_rmsnorm_amd")


def test_earlier_runtime_error_is_not_attributed_to_a_call():
    """A HIP error left by the caller (here hipSetDevice on a device that
    does not exist) must not turn a good call into NORM_ERR_HIP."""
    hip = ctypes.CDLL("libamdhip64.so.7")
    hip.hipSetDevice.argtypes = [ctypes.c_int]
    torch.cuda.set_device(0)
    x = torch.randn(8, 256, device="cuda", dtype=torch.bfloat16)
    w = torch.ones(256, device="cuda", dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert hip.hipSetDevice(1 << 20) != 0  # an error code; nothing launched
    y, rstd = nl.rms_fwd(x, w, 1e-6)  # raises on any nonzero status
    hip.hipGetLastError()  # leave no stale error for torch's own launch checks
    torch.cuda.synchronize()
    assert torch.isfinite(y.float()).all() and torch.isfinite(rstd).all()
