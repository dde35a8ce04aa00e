"""Inputs written by the kernel just before, on the same stream, with no
host synchronisation in between: the depthwise ring kernel (direct-to-LDS
row loads, counted waits) and the staged backward must give the same bits as
a run on settled inputs.  A count of pending memory operations that assumed
stores retire in order with older loads once let a ring row be read before
it had landed, which only showed when the input came from the previous
kernel."""
import pytest
import torch

from depthwise_stencil_implicit_amd import api, synth

from gpu_util import expand_kw

pytestmark = pytest.mark.gpu


def _args(wl):
    kw = expand_kw(wl)
    return api.make_args(transposed=kw["transposed"], groups=kw["groups"], stride=kw["stride"],
                         padding_before=kw["padding_before"], padding_after=kw["padding_after"],
                         dilation=kw["dilation"], output_padding=kw["output_padding"] if kw["transposed"] else None)


def _dw(seed, L, k, s):
    return synth.random_case(seed, rank=2, transposed=False, dtype="bf16", channels_last=True, N=2, C_in=64,
                             C_out=64, groups=64, L=L, k=[k, k], stride=[s, s], padding_before=[k // 2] * 2,
                             padding_after=[k // 2] * 2, dilation=[1, 1], output_padding=[0, 0], has_bias=True)


@pytest.mark.parametrize("wl", [_dw(9700, [256, 258], 3, 1), _dw(9701, [120, 130], 7, 1), _dw(9702, [200, 96], 5, 2),
                                synth.depthwise_bf16_cl(3, 1).with_batch(8)], ids=lambda w: w.name)
def test_depthwise_forward_on_a_just_written_input(wl):
    print(f"fresh input: {wl.name}", flush=True)
    x, w, b = synth.make_inputs(wl, device="cuda")
    prep = api.Prepared(x, w, b, _args(wl))
    ref = prep.empty_output(x.device)
    prep.run(x, w, b, ref)
    torch.cuda.synchronize()
    assert api.kernel_name(prep.plan.kernel) == "dw_cl"
    for i in range(6):
        xf = torch.empty_like(x)
        xf.copy_(x)                      # written by the copy kernel just before
        y = prep.empty_output(x.device)
        prep.run(xf, w, b, y)
        torch.cuda.synchronize()
        n = int((y != ref).sum())
        assert n == 0, f"run {i}: {n} outputs differ from the run on a settled input"


def test_staged_backward_on_a_just_written_gy():
    wl = _dw(9703, [256, 258], 3, 1)
    print(f"fresh gy, staged backward: {wl.name}", flush=True)
    x, w, _ = synth.make_inputs(wl, device="cuda")
    args = _args(wl)
    prep = api.Prepared(x, w, None, args)
    g = torch.Generator().manual_seed(11)
    gy = torch.randn(prep.sizes, generator=g).to(x.dtype).to("cuda").contiguous()
    pb = api.PreparedBackward(x, w, gy, args, need_dw=False, need_db=False)
    assert int(pb.plan.wg_tile[6]) > 0
    ref, _, _ = pb.outputs(gy.device)
    pb.run(x, w, gy, ref, None, None, pb.workspace(gy.device))
    torch.cuda.synchronize()
    for i in range(6):
        dx, _, _ = pb.outputs(gy.device)
        pb.run(x, w, gy, dx, None, None, pb.workspace(gy.device))
        torch.cuda.synchronize()
        n = int((dx != ref).sum())
        assert n == 0, f"run {i}: {n} elements of dx differ from the first run"
