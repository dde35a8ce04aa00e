"""MI355X-native canonical convolution: C ABI library + thin Python binding.

The library (``libmiconv.so``, built from ``csrc/`` by ``build.py``) is loaded
on first use; importing this package does not touch the GPU.
"""
from .api import (ConvError, Prepared, PreparedBackward, _convolution, conv, conv1d, conv2d, conv3d, conv_backward,
                  conv_bind, conv_plan_candidates, conv_plan_tuned,
                  conv_out_shape, conv_plan, conv_run, conv_transpose1d, conv_transpose2d,
                  conv_transpose3d, convolution, describe, kernel_name, make_args, tensor_desc)

__all__ = ["ConvError", "Prepared", "PreparedBackward", "conv", "conv_backward", "conv_plan_candidates",
           "conv_plan_tuned", "conv1d", "conv2d", "conv3d", "conv_transpose1d",
           "conv_transpose2d", "conv_transpose3d", "convolution", "_convolution", "conv_bind",
           "conv_out_shape", "conv_plan", "conv_run", "describe", "kernel_name", "make_args",
           "tensor_desc"]
