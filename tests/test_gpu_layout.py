"""Output layout against torch's own GPU convolution (ATen on ROCm).

The pages define the op's output layout as the one ATen's convolution
returns (executorch PR #25084, "Add triton::convolution and the conv routing
framework", description).  Here torch's GPU convolution runs the same call
shapes and layouts -- 1-D NCL / NLC, 2-D NCHW / NHWC, 3-D NCDHW / NDHWC,
forward and transposed, channels-last weights, and the five measured
workloads at their channel and spatial sizes (batch 2, except the small
depthwise one) -- and its output strides must equal both the reference's rule
(``oracle.out_strides``) and the library's ``conv_out_shape``.

torch's transposed and forward overloads take one symmetric padding, so the
calls use that; the layout depends only on the output sizes and on x's and
w's layouts, which are the workloads' own.
"""
import pytest
import torch
import torch.nn.functional as F

import oracle
from depthwise_stencil_implicit_amd import api, synth

pytestmark = pytest.mark.gpu

BF, H, F32 = torch.bfloat16, torch.float16, torch.float32

# name, x shape, x channels-last, w shape, w channels-last, dtype, transposed, torch kwargs
CASES = [
    ("1d_nlc_fwd", (2, 8, 20), True, (6, 8, 3), False, BF, False, dict(padding=1)),
    ("1d_ncl_fwd", (2, 8, 20), False, (6, 8, 3), False, BF, False, dict(padding=1)),
    ("1d_nlc_T", (2, 8, 20), True, (8, 6, 4), False, BF, True, dict(stride=2, padding=1)),
    ("1d_ncl_T", (2, 8, 20), False, (8, 6, 4), False, F32, True, dict(stride=2, padding=1)),
    ("1d_w_nlc_fwd", (2, 8, 20), False, (6, 8, 3), True, BF, False, dict(padding=1)),
    ("1d_nlc_grouped", (2, 8, 20), True, (8, 2, 3), False, H, False, dict(padding=1, groups=4)),
    ("2d_nhwc_fwd", (2, 8, 9, 10), True, (6, 8, 3, 3), False, BF, False, dict(padding=1)),
    ("2d_nchw_fwd", (2, 8, 9, 10), False, (6, 8, 3, 3), False, BF, False, dict(padding=1)),
    ("2d_w_nhwc_fwd", (2, 8, 9, 10), False, (6, 8, 3, 3), True, F32, False, dict(padding=1)),
    ("2d_nhwc_T", (2, 8, 9, 10), True, (8, 6, 3, 3), False, BF, True, dict(stride=2, padding=1)),
    ("2d_nhwc_depthwise", (2, 8, 9, 10), True, (8, 1, 3, 3), False, H, False, dict(padding=1, groups=8)),
    ("3d_ndhwc_fwd", (2, 8, 5, 6, 7), True, (6, 8, 3, 3, 3), False, BF, False, dict(padding=1)),
    ("3d_ncdhw_fwd", (2, 8, 5, 6, 7), False, (6, 8, 3, 3, 3), False, BF, False, dict(padding=1)),
    ("3d_ndhwc_T", (2, 8, 5, 6, 7), True, (8, 6, 3, 3, 3), False, F32, True, dict(stride=2, padding=1)),
    ("3d_w_ndhwc_fwd", (2, 8, 5, 6, 7), False, (6, 8, 3, 3, 3), True, BF, False, dict(padding=1)),
    # The five measured workloads (batch reduced to 2 where it is larger).
    ("dw_f32_small", (1, 32, 32, 32), False, (32, 1, 3, 3), False, F32, False, dict(padding=1, groups=32)),
    ("dw_bf16_cl", (2, 256, 56, 56), True, (256, 1, 7, 7), False, BF, False, dict(padding=3, groups=256)),
    ("grp_f16", (2, 256, 28, 28), False, (512, 4, 3, 3), False, H, False, dict(padding=1, groups=64)),
    ("dense_bf16", (2, 256, 56, 56), True, (256, 256, 3, 3), False, BF, False, dict(padding=1)),
    ("convT1d_bf16", (2, 512, 8192), True, (512, 512, 4), False, BF, True, dict(stride=2, padding=1)),
]

FWD = {3: F.conv1d, 4: F.conv2d, 5: F.conv3d}
TRN = {3: F.conv_transpose1d, 4: F.conv_transpose2d, 5: F.conv_transpose3d}


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_output_strides_match_torch_gpu(case):
    name, xs, xcl, ws, wcl, dt, transposed, kw = case
    print(f"layout {name}", flush=True)
    g = torch.Generator().manual_seed(0)
    x = torch.randn(xs, generator=g).to(dt)
    w = torch.randn(ws, generator=g).to(dt)
    if xcl:
        x = synth.channels_last_copy(x)
    if wcl:
        w = synth.channels_last_copy(w)
    x, w = x.cuda(), w.cuda()
    y = (TRN if transposed else FWD)[x.dim()](x, w, **kw)
    torch.cuda.synchronize()
    # The reference's rule.
    assert oracle.out_strides(tuple(y.shape), tuple(x.shape), tuple(x.stride()), tuple(w.shape),
                              tuple(w.stride())) == tuple(y.stride()), name
    # The library's layout for the same call.
    p = kw.get("padding", 0)
    args = api.make_args(transposed=transposed, groups=kw.get("groups", 1), stride=kw.get("stride", 1),
                         padding_before=p, padding_after=p)
    d = api.conv_bind(api.describe(x), api.describe(w), None, args)
    sizes, strides = api.conv_out_shape(d)
    assert sizes == tuple(y.shape), name
    assert strides == tuple(y.stride()), name
