"""conv_run_noalloc: the implicit GEMM's workspace taken from the library's
fixed device array instead of the caller's, against conv_run on the same
plan and inputs (the same kernels, so the outputs must be identical), on two
calls in a row -- the second smaller than the first -- and the refusal of a
plan whose workspace exceeds the array."""
import ctypes

import pytest
import torch

from depthwise_stencil_implicit_amd import _abi as A
from depthwise_stencil_implicit_amd import api, synth

pytestmark = pytest.mark.gpu


def _cases():
    # A dense call whose last rows run as split-K tiles (repacked weights and
    # fp32 partial sums in the scratch), then a smaller transposed call.
    big = synth.random_case(9101, rank=2, transposed=False, dtype="bf16", channels_last=True, N=22, C_in=256,
                            C_out=256, groups=1, L=[56, 56], k=[3, 3], stride=[1, 1], padding_before=[1, 1],
                            padding_after=[1, 1], dilation=[1, 1], output_padding=[0, 0], has_bias=True)
    small = synth.random_case(9102, rank=1, transposed=True, dtype="f16", channels_last=True, N=2, C_in=96,
                              C_out=40, groups=1, L=[300], k=[4], stride=[2], padding_before=[1],
                              padding_after=[2], dilation=[1], output_padding=[0], has_bias=True)
    return [big, small]


def _prepare(wl):
    x, w, b = synth.make_inputs(wl, device="cuda")
    r = len(wl.x_shape) - 2
    ex = lambda v: tuple(v) * r if len(v) == 1 else tuple(v)
    args = api.make_args(transposed=wl.transposed, groups=wl.groups, stride=ex(wl.stride),
                         padding_before=ex(wl.padding_before), padding_after=ex(wl.padding_after),
                         dilation=ex(wl.dilation), output_padding=ex(wl.output_padding) if wl.transposed else None)
    return x, w, b, api.Prepared(x, w, b, args)


def test_noalloc_matches_conv_run_on_two_calls():
    lib = A.lib()
    stream = torch.cuda.current_stream().cuda_stream
    sizes = []
    for wl in _cases():
        print(f"no-alloc: {wl.name} x{wl.x_shape} w{wl.w_shape}", flush=True)
        x, w, b, prep = _prepare(wl)
        assert 0 < prep.plan.workspace_bytes <= A.NOALLOC_SCRATCH_BYTES
        sizes.append(prep.plan.workspace_bytes)
        y_ref = prep.empty_output(x.device)
        prep.run(x, w, b, y_ref, prep.workspace(x.device))
        y = prep.empty_output(x.device).fill_(float("nan"))
        st = lib.conv_run_noalloc(ctypes.byref(prep.plan), x.data_ptr(), w.data_ptr(),
                                  b.data_ptr() if b is not None else None, y.data_ptr(), stream)
        assert st == A.OK, api.ConvError(st)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16)), wl.name
    assert sizes[1] < sizes[0]


def test_noalloc_refuses_a_workspace_beyond_its_array():
    lib = A.lib()
    x = torch.empty((1, 4096, 3, 3), dtype=torch.bfloat16, device="cuda")
    w = torch.empty((4096, 4096, 3, 3), dtype=torch.bfloat16, device="cuda")
    prep = api.Prepared(x, w, None, api.make_args(padding_before=1, padding_after=1))
    assert prep.plan.workspace_bytes > A.NOALLOC_SCRATCH_BYTES
    y = prep.empty_output(x.device)
    st = lib.conv_run_noalloc(ctypes.byref(prep.plan), x.data_ptr(), w.data_ptr(), None, y.data_ptr(),
                              torch.cuda.current_stream().cuda_stream)
    assert st == A.ENOSPACE
    assert "scratch" in lib.conv_status_string(st).decode()


def test_noalloc_without_workspace_is_conv_run():
    wl = synth.depthwise_bf16_cl(5, 2).with_batch(2)
    x, w, b, prep = _prepare(wl)
    assert prep.plan.workspace_bytes == 0
    y_ref = prep.empty_output(x.device)
    prep.run(x, w, b, y_ref)
    y = prep.empty_output(x.device)
    st = A.lib().conv_run_noalloc(ctypes.byref(prep.plan), x.data_ptr(), w.data_ptr(), b.data_ptr(),
                                  y.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert st == A.OK
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16))
