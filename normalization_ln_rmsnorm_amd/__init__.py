"""MI355X-native (gfx950) LayerNorm, RMSNorm and BatchNorm.

The compute lives in libmi355norm.so (hand-written HIP kernels behind a C
ABI, see include/mi355norm.h); ``normlib`` is the Python binding over it and
``layers`` the drop-in PyTorch modules (LayerNorm, RMSNorm, BatchNorm1d,
BatchNorm2d with a fused residual add and activation) built on it.
"""
from .normlib import (ACT, NormError, act_dropout_bwd, act_dropout_fwd, bn_bwd, bn_force_path,
                      bn_fwd_eval, bn_fwd_train, bn_shape,
                      bn_workspace_bytes, last_kernels, lib, ln_bwd,
                      ln_bwd_workspace_bytes, ln_fwd, rms_bwd, rms_bwd_noalloc, rms_bwd_workspace_bytes,
                      rms_fwd, arm_kernel_events)
from .layers import (ActDropout, BatchNorm1d, BatchNorm2d, LayerNorm, RMSNorm, output_dtype,
                     parse_act)

__all__ = ["ACT", "NormError", "act_dropout_bwd", "act_dropout_fwd", "bn_bwd", "bn_force_path",
           "bn_fwd_eval", "bn_fwd_train", "bn_shape",
           "bn_workspace_bytes", "last_kernels", "lib", "ln_bwd", "ln_bwd_workspace_bytes",
           "ln_fwd", "rms_bwd", "rms_bwd_noalloc", "rms_bwd_workspace_bytes", "rms_fwd", "arm_kernel_events",
           "ActDropout", "BatchNorm1d", "BatchNorm2d", "LayerNorm", "RMSNorm", "output_dtype",
           "parse_act"]
