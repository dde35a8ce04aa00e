"""HIP graph capture of the library's launches.

conv_run launches only kernels on the caller's stream (no memsets, no
allocations, no synchronisation), so a sequence of calls can be captured in a
HIP graph and replayed.  Here calls on every forward kernel family -- the
depthwise ring stencil, the grouped matrix-core stencil, the dense implicit
GEMM with its weight repack, split-K tail and reduction, the both-phases
transposed kernel and the phase-split transposed tile -- are captured once and
replayed several times, with the program's own eager work and
synchronisations between the replays; every replay must reproduce the eager
result bit for bit (the kernels are deterministic).
"""
import pytest
import torch

from depthwise_stencil_implicit_amd import api, synth

from gpu_util import expand_kw

pytestmark = pytest.mark.gpu


def _prep(wl, force_kernel=None, force_variant=None):
    x, w, b = synth.make_inputs(wl, device="cuda")
    kw = expand_kw(wl)
    args = api.make_args(transposed=kw["transposed"], groups=kw["groups"], stride=kw["stride"],
                         padding_before=kw["padding_before"], padding_after=kw["padding_after"],
                         dilation=kw["dilation"], output_padding=kw["output_padding"] if kw["transposed"] else None)
    p = api.Prepared(x, w, b, args, force_kernel=force_kernel, force_variant=force_variant)
    return p, x, w, b, p.empty_output(x.device), p.workspace(x.device)


def _calls():
    # 17 x 64 x 64 rows: 272 row tiles of 256, the last 16 split over K.
    dense = synth.random_case(7800, rank=2, transposed=False, dtype="bf16", channels_last=True, N=17, C_in=32,
                              C_out=256, groups=1, L=[64, 64], k=[3, 3], stride=[1, 1], padding_before=[1, 1],
                              padding_after=[1, 1], dilation=[1, 1], output_padding=[0, 0], has_bias=True)
    return [
        _prep(synth.depthwise_bf16_cl(7, 1).with_batch(2)),
        _prep(synth.grouped_f16().with_batch(2)),
        _prep(dense),
        _prep(synth.transposed_bf16_nlc().with_batch(1)),
        _prep(synth.transposed_bf16_nlc().with_batch(1), force_kernel="igemm_t", force_variant=0),
    ]


def test_graph_replays_match_eager():
    calls = _calls()
    names = [api.kernel_name(p.plan.kernel) + f"/{int(p.plan.variant)}" for p, *_ in calls]
    print("graph calls:", names, flush=True)
    # The dense call's plan splits its last rows over K (a tail launch and a reduction).
    assert any(int(p.plan.tile[7]) != 0 for p, *_ in calls if api.kernel_name(p.plan.kernel) == "igemm")
    for p, x, w, b, y, ws in calls:
        p.run(x, w, b, y, ws)
    torch.cuda.synchronize()
    ref = [y.clone() for *_, y, _ in calls]

    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        sp = torch.cuda.current_stream().cuda_stream
        for p, x, w, b, y, ws in calls:
            p.run(x, w, b, y, ws, sp)
    for rep in range(4):
        for *_, y, _ in calls:
            y.fill_(float("nan"))
        # the program's own eager work between replays
        p0, x0, w0, b0, y0, ws0 = calls[2]
        scratch = torch.empty_like(y0)
        p0.run(x0, w0, b0, scratch, ws0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, (*_, y, _), r in zip(names, calls, ref):
            assert torch.equal(y, r), f"replay {rep}: {name} differs from the eager result"
