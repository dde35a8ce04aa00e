"""GPU parity of the gradients (conv_plan_backward / conv_run_backward)
against the double-precision reference (oracle.conv_backward), element by
element: |g_gpu - g| <= eps * A + tiny with A the sum of the absolute values
of the element's terms (eps = 1e-6 fp32, 2^-11 fp16, 2^-8 bf16; tiny = half
the gradient dtype's subnormal spacing)."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from depthwise_stencil_implicit_amd import _abi as A
from depthwise_stencil_implicit_amd import api, synth

from gpu_util import EPS, TINY, expand_kw

pytestmark = pytest.mark.gpu


def _args(wl):
    kw = expand_kw(wl)
    return api.make_args(transposed=kw["transposed"], groups=kw["groups"], stride=kw["stride"],
                         padding_before=kw["padding_before"], padding_after=kw["padding_after"],
                         dilation=kw["dilation"], output_padding=kw["output_padding"] if kw["transposed"] else None)


def _gy_for(wl, x, w, seed):
    """A seeded output gradient in y's own layout."""
    prep = api.Prepared(x, w, None, _args(wl))
    g = torch.Generator().manual_seed(seed)
    vals = torch.randn(prep.sizes, generator=g).to(x.dtype)
    gy = torch.empty_strided(prep.sizes, prep.strides, dtype=x.dtype, device=x.device)
    gy.copy_(vals)
    return gy


def _close(got, ref, bound, eps, what):
    g = got.detach().double().cpu().numpy()
    assert g.shape == ref.shape, (what, g.shape, ref.shape)
    bad = ~(np.abs(g - ref) <= eps * bound + TINY[got.dtype])
    if bad.any():
        idx = np.argwhere(bad)[:4]
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outside the bound, e.g. "
                             + "; ".join(f"{tuple(i)} gpu={g[tuple(i)]} ref={ref[tuple(i)]} A={bound[tuple(i)]}"
                                         for i in idx))


def check_backward(wl, seed=0, need=(True, True, True)):
    x, w, b = synth.make_inputs(wl, device="cuda")
    gy = _gy_for(wl, x, w, seed)
    prep = api.PreparedBackward(x, w, gy, _args(wl), need_dx=need[0], need_dw=need[1], need_db=need[2])
    dx, dw, db = prep.outputs(gy.device)
    prep.run(x, w, gy, dx, dw, db, prep.workspace(gy.device))
    torch.cuda.synchronize()
    f = lambda t: t.detach().double().cpu().contiguous().numpy()
    rdx, Adx, rdw, Adw, rdb, Adb = oracle.conv_backward(f(x), f(w), f(gy), **expand_kw(wl))
    eps = EPS[wl.dtype]
    if need[0]:
        _close(dx, rdx, Adx, eps, f"{wl.name} dx")
    if need[1]:
        _close(dw, rdw, Adw, eps, f"{wl.name} dw")
    if need[2]:
        _close(db, rdb, Adb, eps, f"{wl.name} db")
    return prep, (dx, dw, db)


def _desc(wl):
    kw = expand_kw(wl)
    return (f"{wl.name} {wl.dtype} x{wl.x_shape} w{wl.w_shape} cl={wl.channels_last} g={wl.groups} "
            f"s={kw['stride']} pb={kw['padding_before']} pa={kw['padding_after']} d={kw['dilation']} "
            f"op={kw['output_padding']} T={wl.transposed}")


WORKLOADS = [synth.depthwise_f32_small(), synth.depthwise_bf16_cl(3, 1).with_batch(2),
             synth.depthwise_bf16_cl(5, 2).with_batch(2), synth.grouped_f16().with_batch(2),
             synth.dense_bf16_cl().with_batch(2), synth.transposed_bf16_nlc().with_batch(1)]


@pytest.mark.parametrize("wl", WORKLOADS, ids=lambda w: w.name)
def test_workload_gradients(wl):
    """Every element of dx, dw and db of the measured workloads (batch
    reduced so the reference finishes in seconds)."""
    print(f"gradients: {_desc(wl)}", flush=True)
    prep, _ = check_backward(wl, seed=1)
    if wl.name.startswith("dense"):
        assert int(prep.plan.wg_tile[0]) & 1, "the dense call's weight gradient runs on the matrix cores"


def _cases(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        i = len(out)
        transposed = bool(i % 2)
        r = int(rng.integers(1, 4))
        dtype = ["f32", "f16", "bf16"][i % 3]
        groups = int(rng.choice([1, 1, 2, 3]))
        cig = int(rng.choice([1, 3, 8, 16]))
        cog = int(rng.choice([1, 5, 8, 24]))
        L = [int(rng.integers(3, 10 if r < 3 else 6)) for _ in range(r)]
        k = [int(rng.integers(1, 4)) for _ in range(r)]
        s = [int(rng.integers(1, 4)) for _ in range(r)]
        d = [int(rng.integers(1, 3)) for _ in range(r)]
        pb = [int(rng.integers(0, 3)) for _ in range(r)]
        pa = [int(rng.integers(0, 3)) for _ in range(r)]
        op = [int(rng.integers(0, si)) if transposed else 0 for si in s]
        if transposed:
            ok = all((Li - 1) * si + di * (ki - 1) + 1 + opi - pbi - pai >= 1
                     for Li, si, di, ki, pbi, pai, opi in zip(L, s, d, k, pb, pa, op))
        else:
            ok = all(Li + pbi + pai - di * (ki - 1) - 1 >= 0 for Li, pbi, pai, di, ki in zip(L, pb, pa, d, k))
        if not ok:
            continue
        out.append(synth.random_case(8000 + i + 100 * seed, rank=r, transposed=transposed, dtype=dtype,
                                     channels_last=bool(rng.integers(0, 2)), N=int(rng.integers(1, 3)),
                                     C_in=groups * cig, C_out=groups * cog, groups=groups, L=L, k=k, stride=s,
                                     padding_before=pb, padding_after=pa, dilation=d, output_padding=op,
                                     has_bias=False))
    return out


@pytest.mark.parametrize("wl", _cases(30, 1), ids=lambda w: w.name)
def test_gradient_sweep(wl):
    """Forward and transposed calls of every rank, groups, strides,
    dilation, asymmetric padding, output_padding, every dtype, both layouts
    (the matrix-core weight gradient where channels come in 16-byte
    chunks, the simple kernel elsewhere)."""
    print(f"gradient sweep: {_desc(wl)}", flush=True)
    check_backward(wl, seed=2)


def test_matrix_core_weight_gradient_ragged_channels():
    """The matrix-core weight gradient on channel counts that are not
    multiples of its 128-wide tiles, with several ranges of positions and a
    partial last step of 32 positions, forward and transposed."""
    for i, tr in enumerate((False, True)):
        wl = synth.random_case(8900 + i, rank=2, transposed=tr, dtype="bf16", channels_last=True, N=4, C_in=136,
                               C_out=72, groups=1, L=[31, 29] if not tr else [15, 13], k=[3, 2], stride=[2, 1], padding_before=[1, 0],
                               padding_after=[1, 1], dilation=[1, 2], output_padding=[1, 0] if tr else [0, 0],
                               has_bias=False)
        print(f"wgrad mfma ragged: {_desc(wl)}", flush=True)
        prep, _ = check_backward(wl, seed=3)
        assert int(prep.plan.wg_tile[0]) & 1 and int(prep.plan.wg_tile[3]) > 1


def test_selected_gradients_only():
    wl = synth.dense_bf16_cl().with_batch(1)
    for need in ((True, False, False), (False, True, False), (False, False, True)):
        prep, outs = check_backward(wl, seed=4, need=need)
        assert [o is not None for o in outs] == list(need)


def test_empty_batch_gives_zero_weight_and_bias_gradients():
    x = torch.empty((0, 16, 6, 6), dtype=torch.bfloat16, device="cuda")
    w = torch.randn((8, 16, 3, 3), device="cuda").to(torch.bfloat16)
    gy = torch.empty((0, 8, 4, 4), dtype=torch.bfloat16, device="cuda")
    dx, dw, db = api.conv_backward(x, w, gy)
    torch.cuda.synchronize()
    assert dx.shape == x.shape and torch.count_nonzero(dw).item() == 0 and torch.count_nonzero(db).item() == 0


def test_misaligned_operands_use_the_simple_weight_gradient():
    """x at an odd element offset defeats the 16-byte loads of the
    matrix-core weight gradient; the run falls back to the simple kernel and
    stays correct."""
    wl = synth.random_case(8950, rank=2, transposed=False, dtype="f16", channels_last=True, N=2, C_in=32, C_out=40,
                           groups=1, L=[9, 7], k=[3, 3], stride=[1, 1], padding_before=[1, 1],
                           padding_after=[1, 1], dilation=[1, 1], output_padding=[0, 0], has_bias=False)
    x0, w, _ = synth.make_inputs(wl, device="cuda")
    buf = torch.zeros(x0.numel() + 8, dtype=x0.dtype, device="cuda")
    x = torch.as_strided(buf, x0.shape, x0.stride(), 1)
    x.copy_(x0)
    gy = _gy_for(wl, x0, w, 5)
    prep = api.PreparedBackward(x, w, gy, _args(wl))
    assert int(prep.plan.wg_tile[0]) == 1
    dx, dw, db = prep.outputs(gy.device)
    prep.run(x, w, gy, dx, dw, db, prep.workspace(gy.device))
    torch.cuda.synchronize()
    f = lambda t: t.detach().double().cpu().contiguous().numpy()
    _, _, rdw, Adw, _, _ = oracle.conv_backward(f(x), f(w), f(gy), **expand_kw(wl))
    _close(dw, rdw, Adw, EPS["f16"], "misaligned dw")


def _flip_cases():
    """Stride-1 calls whose input gradient runs as the forward call of gy
    with the reversed, channel-exchanged weight on the stencils: depthwise
    channels-last 3x3 / 5x5 / 7x7 (asymmetric padding), channel multiplier 2,
    few-channel grouped NCHW, 1-D NLC and fp32 NCHW."""
    mk = synth.random_case
    return [
        mk(8700, rank=2, transposed=False, dtype="bf16", channels_last=True, N=2, C_in=64, C_out=64, groups=64,
           L=[17, 23], k=[5, 5], stride=[1, 1], padding_before=[2, 2], padding_after=[2, 2], dilation=[1, 1],
           output_padding=[0, 0], has_bias=False),
        mk(8701, rank=2, transposed=False, dtype="bf16", channels_last=True, N=2, C_in=64, C_out=64, groups=64,
           L=[16, 19], k=[7, 7], stride=[1, 1], padding_before=[3, 3], padding_after=[3, 3], dilation=[1, 1],
           output_padding=[0, 0], has_bias=False),
        mk(8702, rank=2, transposed=False, dtype="f16", channels_last=True, N=2, C_in=32, C_out=32, groups=32,
           L=[13, 11], k=[3, 3], stride=[1, 1], padding_before=[0, 2], padding_after=[2, 1], dilation=[1, 1],
           output_padding=[0, 0], has_bias=False),
        mk(8703, rank=2, transposed=False, dtype="bf16", channels_last=True, N=2, C_in=32, C_out=64, groups=32,
           L=[12, 14], k=[3, 3], stride=[1, 1], padding_before=[1, 1], padding_after=[1, 1], dilation=[1, 1],
           output_padding=[0, 0], has_bias=False),
        mk(8704, rank=2, transposed=False, dtype="f16", channels_last=False, N=2, C_in=32, C_out=64, groups=8,
           L=[14, 14], k=[3, 3], stride=[1, 1], padding_before=[1, 1], padding_after=[1, 1], dilation=[1, 1],
           output_padding=[0, 0], has_bias=False),
        mk(8705, rank=1, transposed=False, dtype="bf16", channels_last=True, N=2, C_in=48, C_out=48, groups=48,
           L=[40], k=[7], stride=[1], padding_before=[3], padding_after=[3], dilation=[1], output_padding=[0],
           has_bias=False),
        mk(8706, rank=2, transposed=False, dtype="f32", channels_last=False, N=1, C_in=16, C_out=16, groups=16,
           L=[20, 18], k=[3, 3], stride=[1, 1], padding_before=[1, 1], padding_after=[1, 1], dilation=[1, 1],
           output_padding=[0, 0], has_bias=False),
    ]


@pytest.mark.parametrize("wl", _flip_cases(), ids=lambda w: w.name)
def test_stride1_input_gradient_on_the_stencils(wl):
    """dx of stride-1 depthwise and few-channel grouped calls: the reversed
    weight copied into the workspace, then the forward stencil on gy; every
    element against the reference, and dw / db alongside."""
    print(f"flipped-weight input gradient: {_desc(wl)}", flush=True)
    prep, _ = check_backward(wl, seed=6)
    assert int(prep.plan.dgrad_flip) == 1
    assert api.kernel_name(prep.plan.dgrad.kernel) in ("dw_cl", "plane", "grp", "reduce")


def _dw_wgrad_cases():
    """Depthwise weight gradients on the channel-word stencil: channel counts
    that are not multiples of its 64-channel workgroups, strides 1-2,
    dilation, asymmetric padding, 1x7 to 9x9 (up to 11 taps per thread)."""
    mk = synth.random_case
    return [
        mk(8800, rank=2, transposed=False, dtype="bf16", channels_last=True, N=2, C_in=40, C_out=40, groups=40,
           L=[15, 17], k=[3, 3], stride=[2, 2], padding_before=[0, 1], padding_after=[1, 1], dilation=[1, 1],
           output_padding=[0, 0], has_bias=False),
        mk(8801, rank=2, transposed=False, dtype="f16", channels_last=True, N=3, C_in=96, C_out=96, groups=96,
           L=[14, 12], k=[5, 3], stride=[1, 2], padding_before=[2, 1], padding_after=[2, 0], dilation=[2, 1],
           output_padding=[0, 0], has_bias=False),
        mk(8802, rank=2, transposed=False, dtype="bf16", channels_last=True, N=1, C_in=130, C_out=130, groups=130,
           L=[20, 21], k=[9, 9], stride=[1, 1], padding_before=[4, 4], padding_after=[4, 4], dilation=[1, 1],
           output_padding=[0, 0], has_bias=False),
        mk(8803, rank=2, transposed=False, dtype="bf16", channels_last=True, N=2, C_in=64, C_out=64, groups=64,
           L=[6, 50], k=[1, 7], stride=[1, 2], padding_before=[0, 2], padding_after=[0, 3], dilation=[1, 1],
           output_padding=[0, 0], has_bias=False),
    ]


@pytest.mark.parametrize("wl", _dw_wgrad_cases(), ids=lambda w: w.name)
def test_depthwise_weight_gradient_stencil(wl):
    """Every element of dw (and db) against the reference, on the depthwise
    weight-gradient stencil (fp32 partial sums per range of rows, reduced
    and rounded once)."""
    print(f"depthwise weight gradient: {_desc(wl)}", flush=True)
    prep, _ = check_backward(wl, seed=7, need=(False, True, True))
    assert int(prep.plan.wg_tile[0]) == 8


def _staged_cases():
    """Channels-last x with a channel-major gy of at least 16 MiB: depthwise
    3x3, a transposed 1-D call with 72 output channels (a ragged 64-channel
    tile) and a dense f16 3x3 with 80 output channels."""
    mk = synth.random_case
    return [
        mk(8960, rank=2, transposed=False, dtype="bf16", channels_last=True, N=2, C_in=64, C_out=64, groups=64,
           L=[256, 258], k=[3, 3], stride=[1, 1], padding_before=[1, 1], padding_after=[1, 1], dilation=[1, 1],
           output_padding=[0, 0], has_bias=False),
        mk(8961, rank=1, transposed=True, dtype="bf16", channels_last=True, N=2, C_in=64, C_out=72, groups=1,
           L=[30001], k=[4], stride=[2], padding_before=[1], padding_after=[1], dilation=[1], output_padding=[0],
           has_bias=False),
        mk(8962, rank=2, transposed=False, dtype="f16", channels_last=True, N=2, C_in=32, C_out=80, groups=1,
           L=[210, 250], k=[3, 3], stride=[1, 1], padding_before=[1, 1], padding_after=[1, 1], dilation=[1, 1],
           output_padding=[0, 0], has_bias=False),
    ]


@pytest.mark.parametrize("wl", _staged_cases(), ids=lambda w: w.name)
def test_channel_major_gy_copied_channels_last(wl):
    """A channel-major gy beside channels-last x is first copied
    channels-last into the workspace (a 2-D call's dx then channels-last like
    x, a 1-D call's dx contiguous as before); every
    element of dx, dw and db read from the copy against the reference."""
    print(f"staged gy: {_desc(wl)}", flush=True)
    x, w, _ = synth.make_inputs(wl, device="cuda")
    prep = api.Prepared(x, w, None, _args(wl))
    g = torch.Generator().manual_seed(9)
    gy = torch.randn(prep.sizes, generator=g).to(x.dtype).to("cuda").contiguous()
    pb = api.PreparedBackward(x, w, gy, _args(wl))
    assert int(pb.plan.wg_tile[6]) >= gy.numel() * gy.element_size()
    dx, dw, db = pb.outputs(gy.device)
    assert dx.stride(1) == 1 or x.dim() == 3, "a 2-D call's dx takes x's channels-last layout"
    pb.run(x, w, gy, dx, dw, db, pb.workspace(gy.device))
    torch.cuda.synchronize()
    f = lambda t: t.detach().double().cpu().contiguous().numpy()
    rdx, Adx, rdw, Adw, rdb, Adb = oracle.conv_backward(f(x), f(w), f(gy), **expand_kw(wl))
    eps = EPS[wl.dtype]
    _close(dx, rdx, Adx, eps, f"{wl.name} dx")
    _close(dw, rdw, Adw, eps, f"{wl.name} dw")
    _close(db, rdb, Adb, eps, f"{wl.name} db")
