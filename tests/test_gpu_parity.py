"""GPU parity: the library's kernels against the double-precision reference.

Every comparison is element by element, |y_gpu - y| <= eps * A + tiny with
A = sum|x*w| + |b| (eps = 1e-6 fp32, 2^-11 fp16, 2^-8 bf16; tiny = half the
output dtype's subnormal spacing, the most one rounding can move a result
below the smallest normal number); integer-valued
and all-ones inputs must match exactly.  Output shapes and strides must equal
the reference's layout rule exactly.
"""
import numpy as np
import pytest
import torch

import oracle
from depthwise_stencil_implicit_amd import _abi, api, synth

from gpu_util import EPS, TINY, assert_close, check_full, check_points, expand_kw, ref_inputs, run_gpu

pytestmark = pytest.mark.gpu


def _flush(msg):
    print(msg, flush=True)


# ------------------------------------------------------------ the workloads --

FULL = [synth.depthwise_f32_small()] + synth.depthwise_bf16_cl_all() + [synth.grouped_f16()]


@pytest.mark.parametrize("wl", FULL, ids=lambda w: w.name)
def test_workload_full_output(wl):
    _flush(f"workload {wl.name}")
    y = check_full(wl)
    exp = oracle.out_strides(tuple(y.shape), wl.x_shape,
                             synth.channels_last_copy(torch.empty(wl.x_shape, dtype=torch.int8)).stride()
                             if wl.channels_last else torch.empty(wl.x_shape, dtype=torch.int8).stride(),
                             wl.w_shape, torch.empty(wl.w_shape, dtype=torch.int8).stride())
    assert tuple(y.stride()) == exp


@pytest.mark.parametrize("wl", [synth.dense_bf16_cl(), synth.transposed_bf16_nlc()], ids=lambda w: w.name)
def test_workload_sampled_outputs(wl):
    _flush(f"workload {wl.name} (sampled)")
    y = check_points(wl, n=6000, seed=1)
    exp = oracle.out_strides(tuple(y.shape), wl.x_shape,
                             synth.channels_last_copy(torch.empty(wl.x_shape, dtype=torch.int8)).stride(),
                             wl.w_shape, torch.empty(wl.w_shape, dtype=torch.int8).stride())
    assert tuple(y.stride()) == exp


@pytest.mark.parametrize("wl", [synth.dense_bf16_cl().with_batch(2), synth.transposed_bf16_nlc().with_batch(1)],
                         ids=lambda w: w.name)
def test_workload_reduced_batch_full_output(wl):
    """The same calls at a batch the reference finishes in seconds, whole output."""
    _flush(f"workload {wl.name}")
    check_full(wl)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("wl", [synth.dense_bf16_cl(), synth.transposed_bf16_nlc()], ids=lambda w: w.name)
def test_workload_full_size_whole_output(wl):
    """The dense and transposed workloads at full size, in the launch
    configuration the benchmark times (full-size tiles, and for the dense call
    the split-K rows past the last full round), every output element against
    the reference.  The reference runs a few images at a time to bound host
    memory."""
    _flush(f"workload {wl.name} (whole output, full size)")
    x, w, b, y = run_gpu(wl)
    kw = expand_kw(wl)
    plan = api.Prepared(x, w, b, api.make_args(**{k: v for k, v in kw.items() if k not in ("groups", "transposed")},
                                               groups=wl.groups, transposed=wl.transposed)).plan
    _flush(f"  plan {api.kernel_name(plan.kernel)} variant {plan.variant} tail {int(plan.tile[7])}")
    xr, wr, br = ref_inputs(x, w, b)
    N = x.shape[0]
    step = 8 if not wl.transposed else 2
    for n0 in range(0, N, step):
        n1 = min(N, n0 + step)
        yr, A = oracle.conv(xr[n0:n1], wr, br, **kw)
        assert_close(y[n0:n1], yr, A, EPS[wl.dtype], f"{wl.name} images {n0}..{n1 - 1}")
        _flush(f"  images {n0}..{n1 - 1} ok")


# ----------------------------------------------------------------- sweeps --

def _geom_cases(kind, n, seed):
    rng = np.random.default_rng(seed)
    out = []
    tries = 0
    while len(out) < n and tries < 10000:
        tries += 1
        dtype = ["f32", "f16", "bf16"][len(out) % 3] if kind != "grp" else ["f16", "bf16"][len(out) % 2]
        cl = bool(rng.integers(0, 2))
        bias = bool(rng.integers(0, 2))
        if kind in ("igemm", "igemm_t"):
            r = int(rng.integers(1, 4))
            groups = int(rng.choice([1, 1, 2, 3]))
            cig = int(rng.choice([1, 3, 8, 16, 40]))
            cog = int(rng.choice([1, 5, 16, 33, 70]))
            L = [int(rng.integers(3, 12 if r < 3 else 6)) for _ in range(r)]
            k = [int(rng.integers(1, 4)) for _ in range(r)]
            s = [int(rng.integers(1, 4)) for _ in range(r)]
            d = [int(rng.integers(1, 3)) for _ in range(r)]
            N = int(rng.integers(1, 4))
        else:
            r = int(rng.integers(1, 3))
            cig = int(rng.integers(1, 9)) if kind != "dw_cl" else 1
            mult = int(rng.choice([1, 2, 3, 16, 17])) if kind != "dw_cl" else 1
            groups = int(rng.integers(2, 6)) if kind != "dw_cl" else int(rng.choice([8, 12, 20, 40, 64, 128, 256]))
            cog = mult
            N = int(rng.integers(1, 3))
            if kind == "dw_cl":
                r = 2
                kk = int(rng.choice([3, 5, 7]))
                ss = int(rng.integers(1, 3))
                k, s, d = [kk, kk], [ss, ss], [1, 1]
                L = [int(rng.integers(kk, 20)), int(rng.integers(kk, 40))]
                cl = True
            elif kind == "reduce":
                k = [int(rng.integers(3, 10)) for _ in range(r)]
                s = [int(rng.integers(1, 3)) for _ in range(r)]
                d = [1] * r
                L = [int(rng.integers(kk, kk + 2)) for kk in k]
            else:
                k = [int(rng.integers(1, 10)) for _ in range(r)]
                s = [int(rng.integers(1, 4)) for _ in range(r)]
                d = [int(rng.integers(1, 3)) for _ in range(r)]
                L = [int(rng.integers(max(3, k[i]), 40)) for i in range(r)]
        pb = [int(rng.integers(0, 3)) for _ in range(r)]
        pa = [int(rng.integers(0, 3)) for _ in range(r)]
        transposed = kind == "igemm_t"
        op = [int(rng.integers(0, max(si, di))) if transposed else 0 for si, di in zip(s, d)]
        if transposed:
            ok = all((Li - 1) * si + di * (ki - 1) + 1 + opi - pbi - pai >= 1
                     for Li, si, di, ki, pbi, pai, opi in zip(L, s, d, k, pb, pa, op))
        else:
            ok = all(Li + pbi + pai - di * (ki - 1) - 1 >= 0 for Li, pbi, pai, di, ki in zip(L, pb, pa, d, k))
        if not ok:
            continue
        wl = synth.random_case(1000 + len(out) + 100 * seed, rank=r, transposed=transposed, dtype=dtype,
                               channels_last=cl, N=N, C_in=groups * cig, C_out=groups * cog, groups=groups,
                               L=L, k=k, stride=s, padding_before=pb, padding_after=pa, dilation=d,
                               output_padding=op, has_bias=bias)
        out.append(wl)
    return out


def _grp_flat_cases(n, seed):
    """Grouped calls inside the flat grouped schedule's domain: 3x3 with equal
    strides 1 or 2, or one row of 1, 3, 5 or 7 taps at stride 1 or 2, unit
    dilation; any channel counts, pads, layouts and ragged sizes."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        i = len(out)
        dtype = ["f16", "bf16"][i % 2]
        r = 2 if i % 3 else 1
        ss = int(rng.integers(1, 3))
        if r == 2:
            k = [3, 3] if i % 4 else [1, int(rng.choice([1, 3, 5, 7]))]
            s = [ss, ss] if k[0] == 3 else [int(rng.integers(1, 4)), ss]
            L = [int(rng.integers(3, 30)), int(rng.integers(max(3, k[1]), 70))]
        else:
            k = [int(rng.choice([1, 3, 5, 7]))]
            s = [ss]
            L = [int(rng.integers(k[0], 300))]
        cig = int(rng.integers(1, 9))
        groups = int(rng.integers(2, 7))
        cog = int(rng.choice([1, 2, 3, 8, 9, 16, 17]))
        pb = [int(rng.integers(0, kk)) if kk > 1 else 0 for kk in k]
        pa = [int(rng.integers(0, kk)) if kk > 1 else 0 for kk in k]
        if not all(Li + pbi + pai - (ki - 1) - 1 >= 0 for Li, pbi, pai, ki in zip(L, pb, pa, k)):
            continue
        out.append(synth.random_case(5000 + i + 100 * seed, rank=r, transposed=False, dtype=dtype,
                                     channels_last=bool(rng.integers(0, 2)), N=int(rng.integers(1, 4)),
                                     C_in=groups * cig, C_out=groups * cog, groups=groups, L=L, k=k, stride=s,
                                     padding_before=pb, padding_after=pa, dilation=[1] * r,
                                     output_padding=[0] * r, has_bias=bool(rng.integers(0, 2))))
    return out


GRP_FLAT = _grp_flat_cases(24, 7)


def _grp_plane_cases(n, seed):
    """Grouped 3x3 calls inside the one-plane-per-workgroup schedule's domain:
    contiguous NCHW x and y whose per-group planes are whole 16-byte chunks,
    equal strides 1 or 2, unit dilation, small planes; any pads, channel
    counts (odd ones included) and bias."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        i = len(out)
        s = int(rng.integers(1, 3))
        cig = int(rng.integers(1, 9))
        cog = int(rng.choice([1, 2, 3, 4, 8, 9, 16]))
        groups = int(rng.integers(1, 5)) * 2
        H, W = int(rng.integers(3, 33)), int(rng.integers(3, 33))
        pb = [int(rng.integers(0, 3)) for _ in range(2)]
        pa = [int(rng.integers(0, 3)) for _ in range(2)]
        OH = (H + pb[0] + pa[0] - 3) // s + 1
        OW = (W + pb[1] + pa[1] - 3) // s + 1
        if OH < 1 or OW < 1:
            continue
        N = int(rng.integers(1, 4))
        threads = -(-cog * -(-OH // 2) * -(-OW // 7) // 64) * 64
        if (cig * H * W) % 8 or (cog * OH * OW) % 8 or threads > 512 or -(-(cig * H * W * 2) // 16) > threads:
            continue
        out.append(synth.random_case(6000 + i + 100 * seed, rank=2, transposed=False,
                                     dtype=["f16", "bf16"][i % 2], channels_last=False, N=N,
                                     C_in=groups * cig, C_out=groups * cog, groups=groups, L=[H, W], k=[3, 3],
                                     stride=[s, s], padding_before=pb, padding_after=pa, dilation=[1, 1],
                                     output_padding=[0, 0], has_bias=bool(rng.integers(0, 2))))
    return out


GRP_PLANE = _grp_plane_cases(24, 8)


def _grp_mma_cases(n, seed):
    """Grouped 3x3 calls inside the matrix-core plane schedule's domain:
    contiguous NCHW planes in whole 16-byte (input) and 8-byte (output)
    pieces, output rows of a multiple of 4 columns, up to 16 output
    channels per group, equal strides 1 or 2; odd channel counts and both
    channel-slot widths (Cig <= 4 and 5..8)."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        i = len(out)
        s = int(rng.integers(1, 3))
        cig = int(rng.integers(1, 9))
        cog = int(rng.choice([1, 2, 3, 5, 8, 12, 16]))
        groups = int(rng.integers(1, 6))
        H, W = int(rng.integers(3, 40)), int(rng.integers(3, 40))
        pb = [int(rng.integers(0, 3)) for _ in range(2)]
        pa = [int(rng.integers(0, 3)) for _ in range(2)]
        OH = (H + pb[0] + pa[0] - 3) // s + 1
        OW = (W + pb[1] + pa[1] - 3) // s + 1
        if OH < 1 or OW < 1 or groups * cig < 2:
            continue
        if (cig * H * W) % 8 or OW % 4 or cig * H * W > 4096 or cog * OH * OW > 8192:
            continue
        cp = 4 if cig <= 4 else 8
        IHh, IWh = (OH - 1) * s + 3, (OW - 1) * s + 3
        if IHh * IWh * cp * 2 + cog * OH * OW * 2 + 64 > 64 * 1024:
            continue
        out.append(synth.random_case(7000 + i + 100 * seed, rank=2, transposed=False,
                                     dtype=["f16", "bf16"][i % 2], channels_last=False,
                                     N=int(rng.integers(1, 4)), C_in=groups * cig, C_out=groups * cog,
                                     groups=groups, L=[H, W], k=[3, 3], stride=[s, s], padding_before=pb,
                                     padding_after=pa, dilation=[1, 1], output_padding=[0, 0],
                                     has_bias=bool(rng.integers(0, 2))))
    return out


GRP_MMA = _grp_mma_cases(20, 9)

SWEEP = {kind: _geom_cases(kind, n, seed) for kind, n, seed in
         [("igemm", 24, 1), ("igemm_t", 24, 2), ("plane", 24, 3), ("dw_cl", 24, 4), ("reduce", 9, 5),
          ("grp", 24, 6)]}


def _desc(wl):
    kw = expand_kw(wl)
    return (f"{wl.name} {wl.dtype} x{wl.x_shape} w{wl.w_shape} cl={wl.channels_last} g={wl.groups} "
            f"s={kw['stride']} pb={kw['padding_before']} pa={kw['padding_after']} d={kw['dilation']} "
            f"op={kw['output_padding']} bias={wl.has_bias}")


@pytest.mark.parametrize("kind,wl", [(k, w) for k, ws in SWEEP.items() for w in ws],
                         ids=lambda v: v if isinstance(v, str) else v.name)
def test_forced_kernel_sweep(kind, wl):
    _flush(f"sweep {kind}: {_desc(wl)}")
    check_full(wl, force=kind)


@pytest.mark.parametrize("wl", GRP_FLAT + GRP_PLANE + GRP_MMA, ids=lambda v: v.name)
def test_grp_flat_sweep(wl):
    _flush(f"sweep grp (flat / plane domain): {_desc(wl)}")
    check_full(wl, force="grp")


# ------------------------------------------------------------- exactness --

EXACT_CASES = [
    ("dw_cl", synth.random_case(7, rank=2, transposed=False, dtype="bf16", channels_last=True, N=2, C_in=32,
                                C_out=32, groups=32, L=[13, 21], k=[5, 5], stride=[1, 1],
                                padding_before=[2, 1], padding_after=[1, 2], dilation=[1, 1],
                                output_padding=[0, 0], has_bias=True)),
    ("plane", synth.random_case(8, rank=2, transposed=False, dtype="f16", channels_last=False, N=2, C_in=12,
                                C_out=24, groups=3, L=[17, 19], k=[3, 4], stride=[2, 1],
                                padding_before=[1, 2], padding_after=[0, 1], dilation=[1, 1],
                                output_padding=[0, 0], has_bias=True)),
    ("grp", synth.random_case(12, rank=2, transposed=False, dtype="bf16", channels_last=False, N=2, C_in=20,
                              C_out=40, groups=4, L=[15, 17], k=[3, 3], stride=[1, 2],
                              padding_before=[1, 1], padding_after=[1, 0], dilation=[1, 1],
                              output_padding=[0, 0], has_bias=True)),
    ("grp", synth.random_case(13, rank=1, transposed=False, dtype="f16", channels_last=True, N=3, C_in=14,
                              C_out=21, groups=7, L=[33], k=[5], stride=[1], padding_before=[2],
                              padding_after=[1], dilation=[2], output_padding=[0], has_bias=False)),
    ("grp", synth.random_case(14, rank=2, transposed=False, dtype="f16", channels_last=False, N=3, C_in=15,
                              C_out=45, groups=5, L=[14, 19], k=[3, 3], stride=[2, 2],
                              padding_before=[1, 0], padding_after=[0, 1], dilation=[1, 1],
                              output_padding=[0, 0], has_bias=True)),
    ("igemm", synth.random_case(9, rank=2, transposed=False, dtype="bf16", channels_last=True, N=2, C_in=64,
                                C_out=48, groups=1, L=[9, 10], k=[3, 3], stride=[1, 2],
                                padding_before=[1, 0], padding_after=[2, 1], dilation=[1, 1],
                                output_padding=[0, 0], has_bias=True)),
    ("igemm_t", synth.random_case(10, rank=1, transposed=True, dtype="bf16", channels_last=True, N=2,
                                  C_in=32, C_out=32, groups=1, L=[40], k=[4], stride=[2], padding_before=[1],
                                  padding_after=[2], dilation=[1], output_padding=[0], has_bias=False)),
    ("igemm", synth.random_case(11, rank=3, transposed=False, dtype="f32", channels_last=False, N=1, C_in=6,
                                C_out=10, groups=2, L=[5, 6, 7], k=[2, 3, 2], stride=[1, 2, 1],
                                padding_before=[1, 0, 1], padding_after=[0, 1, 1], dilation=[2, 1, 1],
                                output_padding=[0, 0, 0], has_bias=True)),
]


EXACT_CASES += [
    ("dw_cl", synth.random_case(15, rank=2, transposed=False, dtype="f16", channels_last=True, N=2, C_in=64,
                                C_out=64, groups=64, L=[11, 30], k=[7, 7], stride=[1, 1],
                                padding_before=[3, 3], padding_after=[3, 3], dilation=[1, 1],
                                output_padding=[0, 0], has_bias=True)),
    ("dw_cl", synth.random_case(16, rank=2, transposed=False, dtype="bf16", channels_last=True, N=2, C_in=48,
                                C_out=48, groups=48, L=[12, 33], k=[3, 3], stride=[2, 2],
                                padding_before=[0, 0], padding_after=[1, 1], dilation=[1, 1],
                                output_padding=[0, 0], has_bias=True)),
    ("plane", synth.random_case(17, rank=2, transposed=False, dtype="bf16", channels_last=True, N=2, C_in=16,
                                C_out=16, groups=16, L=[15, 13], k=[5, 5], stride=[1, 1],
                                padding_before=[2, 2], padding_after=[2, 2], dilation=[1, 1],
                                output_padding=[0, 0], has_bias=True)),
    # The grouped matrix-core plane schedule (3x3, NCHW planes, 12 columns).
    ("grp", synth.random_case(18, rank=2, transposed=False, dtype="f16", channels_last=False, N=3, C_in=6,
                              C_out=16, groups=2, L=[8, 12], k=[3, 3], stride=[1, 1],
                              padding_before=[1, 1], padding_after=[1, 1], dilation=[1, 1],
                              output_padding=[0, 0], has_bias=True)),
    ("grp", synth.random_case(19, rank=2, transposed=False, dtype="bf16", channels_last=False, N=3, C_in=8,
                              C_out=10, groups=2, L=[8, 16], k=[3, 3], stride=[2, 2],
                              padding_before=[1, 1], padding_after=[1, 1], dilation=[1, 1],
                              output_padding=[0, 0], has_bias=False)),
]


@pytest.mark.parametrize("kind,wl", EXACT_CASES, ids=lambda v: v if isinstance(v, str) else v.name)
@pytest.mark.parametrize("values", ["ones", "ints", "wide"])
def test_exact_results(kind, wl, values):
    """Integer inputs have exact fp32 sums in any order, so every kernel must
    return the exact sum rounded once, to nearest even, to the output dtype.
    "ones" and "ints" stay small enough to be exact in every dtype; "wide"
    (x in [-127, 127], w in [-31, 31]) gives sums well above 256 (bf16) and
    2048 (fp16) with odd low bits, so each output needs a rounding -- a
    truncating or twice-rounding epilogue fails it."""
    import dataclasses
    if values == "ones":
        wl = dataclasses.replace(wl, x_dist=("ones",), w_dist=("ones",), b_dist=("ones",))
    elif values == "ints":
        wl = dataclasses.replace(wl, x_dist=("ints", -3, 3), w_dist=("ints", -2, 2), b_dist=("ints", -4, 4))
    else:
        wl = dataclasses.replace(wl, x_dist=("ints", -127, 127), w_dist=("ints", -31, 31),
                                 b_dist=("ints", -500, 500))
    _flush(f"exact {values} {kind}: {_desc(wl)}")
    y = check_full(wl, force=kind, exact=True)
    if values == "wide" and wl.dtype != "f32":
        # The case really exercises the rounding: many outputs beyond the
        # range where every integer is representable.
        lim = 256 if wl.dtype == "bf16" else 2048
        assert (y.abs().float() > lim).float().mean().item() > 0.2


# ------------------------------------------------------------ memory safety --

@pytest.mark.parametrize("kind,wl", [(k, ws[i]) for k, ws in SWEEP.items() for i in (0, 1)] +
                         [("grp", GRP_FLAT[i]) for i in (0, 1, 2)] + [("grp", GRP_PLANE[i]) for i in (0, 1, 2)] +
                         [("grp", GRP_MMA[i]) for i in (0, 1, 2)],
                         ids=lambda v: v if isinstance(v, str) else v.name)
def test_writes_stay_inside_output(kind, wl):
    """y sits inside a canary-filled buffer and starts as NaN: afterwards the
    canary is intact and no element of y is left NaN."""
    _flush(f"guard {kind}: {_desc(wl)}")
    x, w, b = synth.make_inputs(wl, device="cuda")
    kw = expand_kw(wl)
    args = api.make_args(transposed=kw["transposed"], groups=kw["groups"], stride=kw["stride"],
                         padding_before=kw["padding_before"], padding_after=kw["padding_after"],
                         dilation=kw["dilation"], output_padding=kw["output_padding"] if kw["transposed"] else None)
    prep = api.Prepared(x, w, b, args, force_kernel=kind)
    numel = int(np.prod(prep.sizes))
    span = 1 + sum((s - 1) * st for s, st in zip(prep.sizes, prep.strides))
    guard = 4096
    buf = torch.full((span + 2 * guard,), 7.0, dtype=x.dtype, device="cuda")
    y = torch.as_strided(buf, prep.sizes, prep.strides, guard)
    y.fill_(float("nan"))
    prep.run(x, w, b, y, prep.workspace(x.device))
    torch.cuda.synchronize()
    assert not torch.isnan(y).any()
    assert (buf[:guard] == 7.0).all() and (buf[guard + span:] == 7.0).all()
    xr, wr, br = ref_inputs(x, w, b)
    yr, A = oracle.conv(xr, wr, br, **kw)
    assert_close(y, yr, A, EPS[wl.dtype], wl.name)
    assert numel == y.numel()


# ------------------------------------------------------------- edge cases --

def test_empty_batch_is_a_noop():
    x = torch.empty((0, 8, 5, 5), dtype=torch.bfloat16, device="cuda")
    w = torch.randn((8, 1, 3, 3), device="cuda").to(torch.bfloat16)
    y = api.conv(x, w, None, groups=8, padding_before=1, padding_after=1)
    assert tuple(y.shape) == (0, 8, 5, 5)


def test_unbatched_and_same_padding():
    g = torch.Generator().manual_seed(3)
    x = torch.randn((6, 11, 9), generator=g).to(torch.float16)
    w = (0.3 * torch.randn((12, 2, 3, 4), generator=g)).to(torch.float16)
    b = torch.randn((12,), generator=g).to(torch.float16)
    y = api.conv2d(x.cuda(), w.cuda(), b.cuda(), padding="same", groups=3)
    torch.cuda.synchronize()
    assert tuple(y.shape) == (12, 11, 9)
    yr, A = oracle.conv(x.double()[None].numpy(), w.double().numpy(), b.double().numpy(),
                        padding_before=(1, 1), padding_after=(1, 2), groups=3)
    assert_close(y[None], yr, A, EPS["f16"], "unbatched same")


def test_misaligned_output_uses_scalar_path():
    """A y view at an odd element offset defeats 16-byte stores; the run must
    still be correct (the launcher falls back to the element-wise path)."""
    wl = synth.depthwise_bf16_cl(3, 1).with_batch(2)
    x, w, b = synth.make_inputs(wl, device="cuda")
    kw = expand_kw(wl)
    args = api.make_args(groups=wl.groups, stride=kw["stride"], padding_before=kw["padding_before"],
                         padding_after=kw["padding_after"])
    prep = api.Prepared(x, w, b, args)
    span = 1 + sum((s - 1) * st for s, st in zip(prep.sizes, prep.strides))
    buf = torch.zeros(span + 1, dtype=x.dtype, device="cuda")
    y = torch.as_strided(buf, prep.sizes, prep.strides, 1)
    prep.run(x, w, b, y)
    torch.cuda.synchronize()
    xr, wr, br = ref_inputs(x, w, b)
    yr, A = oracle.conv(xr, wr, br, **kw)
    assert_close(y, yr, A, EPS["bf16"], "misaligned y")


def test_aten_style_overloads_match_reference():
    g = torch.Generator().manual_seed(5)
    x = torch.randn((2, 4, 10), generator=g).to(torch.bfloat16)
    w = (0.3 * torch.randn((4, 3, 3), generator=g)).to(torch.bfloat16)
    y = api.conv_transpose1d(x.cuda(), w.cuda(), None, stride=2, padding=1, output_padding=1)
    torch.cuda.synchronize()
    yr, A = oracle.conv(x.double().numpy(), w.double().numpy(), None, stride=2, padding_before=1,
                        padding_after=1, transposed=True, output_padding=1)
    assert_close(y, yr, A, EPS["bf16"], "conv_transpose1d")
    y2 = api.convolution(x.cuda(), w.permute(1, 0, 2).contiguous().cuda(), None, [1], [2], [1], False, [0], 1)
    torch.cuda.synchronize()
    yr2, A2 = oracle.conv(x.double().numpy(), w.permute(1, 0, 2).double().numpy(), None, padding_before=2,
                          padding_after=2)
    assert_close(y2, yr2, A2, EPS["bf16"], "convolution")


# ------------------------------------------------ rows past the full rounds --

def _tail_case(transposed):
    if not transposed:
        # 22 x 56 x 56 rows in 256-row tiles: 270 tiles, 14 past one round of
        # 256 CUs -> their rows run as split-K 64-row tiles.
        return synth.random_case(7001, rank=2, transposed=False, dtype="bf16", channels_last=True, N=22,
                                 C_in=256, C_out=256, groups=1, L=[56, 56], k=[3, 3], stride=[1, 1],
                                 padding_before=[1, 1], padding_after=[1, 1], dilation=[1, 1],
                                 output_padding=[0, 0], has_bias=True)
    # Transposed 1-D, stride 2: 2 phases x 32 row tiles x 2 column tiles ...
    return synth.random_case(7002, rank=1, transposed=True, dtype="bf16", channels_last=True, N=1,
                             C_in=512, C_out=512, groups=1, L=[66000], k=[4], stride=[2], padding_before=[1],
                             padding_after=[2], dilation=[1], output_padding=[0], has_bias=True)


@pytest.mark.parametrize("transposed", [False, True], ids=["forward", "transposed"])
def test_tail_rows_split_k(transposed):
    """Calls whose last round of full-size tiles would be sparse: the rows past
    the full rounds (64-row tiles with K split, partial sums reduced with the
    bias) against the reference, sampled densely there and at the boundary."""
    wl = _tail_case(transposed)
    _flush(f"tail rows: {_desc(wl)}")
    # The transposed call runs the phase-split tiles (configuration 0); by
    # default it would take the both-phases kernel, which has tests of its own.
    v = 0 if transposed else None
    x, w, b, y = run_gpu(wl, force="igemm_t" if transposed else None, variant=v)
    plan = api.Prepared(x, w, b, api.make_args(**{k: v for k, v in expand_kw(wl).items()
                                                  if k not in ("groups", "transposed")},
                                               groups=wl.groups, transposed=wl.transposed),
                        force_kernel="igemm_t" if transposed else None, force_variant=v).plan
    tail = int(plan.tile[7])
    if not transposed:
        assert tail != 0 and (tail >> 24) > 1, "shape chosen to exercise the split-K rows"
    xr, wr, br = ref_inputs(x, w, b)
    rng = np.random.default_rng(11)
    shape = tuple(y.shape)
    n = 12000
    pts = np.stack([rng.integers(0, s, n) for s in shape], axis=1)
    # Half the points in the last images / positions (the rows past the full rounds).
    if not transposed:
        pts[: n // 2, 0] = shape[0] - 1 - rng.integers(0, 2, n // 2)
    else:
        pts[: n // 2, 2] = shape[2] - 1 - rng.integers(0, 9000, n // 2)
    yr, A = oracle.conv_points(xr, wr, br, pts, **expand_kw(wl))
    yg = y.detach()[tuple(torch.as_tensor(pts.T, device=y.device))].double().cpu().numpy()
    bad = ~(np.abs(yg - yr) <= EPS[wl.dtype] * A + TINY[y.dtype])
    assert not bad.any(), f"{int(bad.sum())} outputs outside the bound, e.g. {pts[bad][:3].tolist()}"


@pytest.mark.timeout(300)
@pytest.mark.parametrize("transposed", [False, True], ids=["forward", "transposed"])
def test_tail_rows_whole_output(transposed):
    """The same calls, every output element: the 256x256 tile (configuration
    0) over whole rounds of full tiles, and the rows past them (64-row tiles;
    for the forward call their K range split over several workgroups and the
    fp32 partial sums reduced with the bias)."""
    wl = _tail_case(transposed)
    _flush(f"tail rows, whole output: {_desc(wl)}")
    v = 0 if transposed else None
    x, w, b, y = run_gpu(wl, force="igemm_t" if transposed else None, variant=v)
    kw = expand_kw(wl)
    plan = api.Prepared(x, w, b, api.make_args(**{k: v for k, v in kw.items() if k not in ("groups", "transposed")},
                                               groups=wl.groups, transposed=wl.transposed),
                        force_kernel="igemm_t" if transposed else None, force_variant=v).plan
    assert int(plan.variant) == 0, "shape chosen for the 256x256 tile"
    if not transposed:
        assert (int(plan.tile[7]) >> 24) > 1 and (int(plan.tile[7]) & 0xffffff) >= 2
    xr, wr, br = ref_inputs(x, w, b)
    step = 6 if not transposed else 1
    for n0 in range(0, x.shape[0], step):
        n1 = min(x.shape[0], n0 + step)
        yr, A = oracle.conv(xr[n0:n1], wr, br, **kw)
        assert_close(y[n0:n1], yr, A, EPS[wl.dtype], f"{wl.name} images {n0}..{n1 - 1}")


def test_wide_grouped_product_on_the_gemm():
    """Few input channels per group but a wide per-group output: the weights
    would not fit the grouped stencil's LDS, so the call runs on the implicit
    GEMM; whole output against the reference."""
    wl = synth.random_case(7501, rank=2, transposed=False, dtype="f16", channels_last=False, N=2, C_in=16,
                           C_out=2048, groups=2, L=[13, 11], k=[9, 9], stride=[1, 1], padding_before=[4, 4],
                           padding_after=[4, 3], dilation=[1, 1], output_padding=[0, 0], has_bias=True)
    _flush(f"wide grouped: {_desc(wl)}")
    x, w, b = synth.make_inputs(wl, device="cuda")
    kw = expand_kw(wl)
    plan = api.Prepared(x, w, b, api.make_args(**{k: v for k, v in kw.items() if k not in ("groups", "transposed")},
                                               groups=wl.groups, transposed=wl.transposed)).plan
    assert api.kernel_name(plan.kernel) == "igemm"
    check_full(wl)


# ---------------------------------------------- every implicit-GEMM tiling --

def _cfg_cases():
    """16-bit implicit-GEMM calls whose K ranges are 1, 2, 3 and 5 steps of 64
    channels (2, 4, 6 and 10 of 32), so every stage count meets step counts
    below it and ones that are not a multiple of it; plus a transposed call
    and a grouped one with a ragged channel block."""
    out = []
    for i, (cig, k, cog) in enumerate([(64, 1, 16), (128, 1, 70), (64, 3, 33), (320, 1, 5)]):
        out.append(synth.random_case(7100 + i, rank=1, transposed=False, dtype=["bf16", "f16"][i % 2],
                                     channels_last=True, N=2, C_in=cig, C_out=cog, groups=1, L=[37], k=[k],
                                     stride=[1], padding_before=[k // 2], padding_after=[k // 2], dilation=[1],
                                     output_padding=[0], has_bias=bool(i % 2)))
    out.append(synth.random_case(7104, rank=1, transposed=True, dtype="bf16", channels_last=True, N=2, C_in=96,
                                 C_out=40, groups=1, L=[29], k=[4], stride=[2], padding_before=[1],
                                 padding_after=[2], dilation=[1], output_padding=[0], has_bias=True))
    out.append(synth.random_case(7105, rank=2, transposed=False, dtype="f16", channels_last=False, N=1, C_in=2 * 72,
                                 C_out=2 * 24, groups=2, L=[9, 11], k=[3, 3], stride=[1, 2], padding_before=[1, 0],
                                 padding_after=[1, 2], dilation=[1, 1], output_padding=[0, 0], has_bias=False))
    return out


CFG_CASES = _cfg_cases()
# Tile configurations of the 16-bit path (index 5 is the fp32 register-staged
# one); the test checks that the plan took each index.
CFGS_16 = [0, 1, 2, 3, 4, 6, 7, 8, 9, 10, 11]


@pytest.mark.parametrize("cfg", CFGS_16)
@pytest.mark.parametrize("wl", CFG_CASES, ids=lambda v: v.name)
def test_igemm_every_tile_config(wl, cfg):
    """The planner's tile choice forced to every configuration (conv_plan_ex's
    force_variant), whole output against the reference: two-stage tiles, and
    three- and four-stage tiles whose step counts are padded to whole rounds
    with dead refills."""
    kind = "igemm_t" if wl.transposed else "igemm"
    _flush(f"tile config {cfg}: {_desc(wl)}")
    x, w, b = synth.make_inputs(wl, device="cuda")
    kw = expand_kw(wl)
    plan = api.Prepared(x, w, b, api.make_args(**{k: v for k, v in kw.items() if k not in ("groups", "transposed")},
                                               groups=wl.groups, transposed=wl.transposed),
                        force_kernel=kind, force_variant=cfg).plan
    assert int(plan.variant) == cfg, f"the plan did not take tile configuration {cfg}"
    check_full(wl, force=kind, variant=cfg)


def _staged_row_cases():
    """Forward 16-bit calls with dense channels-last outputs, which leave the
    tile through the LDS-staged 16-byte row stores: several full row tiles
    plus a partial one, a partial channel tile, groups (the channel offset of
    each group), bias and none."""
    return [synth.random_case(7150, rank=2, transposed=False, dtype="bf16", channels_last=True, N=1, C_in=64,
                              C_out=264, groups=1, L=[24, 24], k=[3, 3], stride=[1, 1], padding_before=[1, 1],
                              padding_after=[1, 1], dilation=[1, 1], output_padding=[0, 0], has_bias=True),
            synth.random_case(7151, rank=2, transposed=False, dtype="f16", channels_last=True, N=2, C_in=2 * 64,
                              C_out=2 * 136, groups=2, L=[20, 15], k=[3, 3], stride=[1, 1], padding_before=[1, 1],
                              padding_after=[1, 1], dilation=[1, 1], output_padding=[0, 0], has_bias=False)]


@pytest.mark.parametrize("cfg", CFGS_16)
@pytest.mark.parametrize("wl", _staged_row_cases(), ids=lambda v: v.name)
def test_igemm_staged_output_rows(wl, cfg):
    """Every tile configuration on outputs whose rows are linear in y: the
    tile is staged in LDS (in two passes where the stages hold fewer rows
    than the tile) and written as whole 16-byte chunks; whole output against
    the reference, and y's layout is the dense channels-last one this path
    needs."""
    _flush(f"staged rows, tile config {cfg}: {_desc(wl)}")
    y = check_full(wl, force="igemm", variant=cfg)
    assert y.stride(1) == 1 and y.stride(-1) == y.shape[1]


# ------------------------------------------- every depthwise ring kernel --

def _dw_every_case():
    """One channels-last depthwise call per compiled ring kernel: kernel 3, 5,
    7 and 9, stride 1 and 2, fp32 / fp16 / bf16, channel runs of whole 16-byte
    chunks (the 16-byte path) and not (the 4-byte path; 12 channels of 16-bit
    or 6 of fp32 are 24 bytes), asymmetric padding and a ragged column chunk
    (72 output columns at stride 1, more than one 56-column chunk)."""
    out = []
    i = 0
    for k in (3, 5, 7, 9):
        for s in (1, 2):
            for dtype in ("f32", "f16", "bf16"):
                for aligned in (True, False):
                    es = 4 if dtype == "f32" else 2
                    C = (64 // es) if aligned else (24 // es)
                    W = 72 * s + k
                    out.append(synth.random_case(7300 + i, rank=2, transposed=False, dtype=dtype,
                                                 channels_last=True, N=2, C_in=C, C_out=C, groups=C,
                                                 L=[9 + k, W], k=[k, k], stride=[s, s],
                                                 padding_before=[k // 2, max(0, k // 2 - 1)],
                                                 padding_after=[k // 2, k // 2], dilation=[1, 1],
                                                 output_padding=[0, 0], has_bias=bool(i % 2)))
                    i += 1
    return out


@pytest.mark.parametrize("wl", _dw_every_case(), ids=lambda v: v.name)
def test_dw_cl_every_ring_kernel(wl):
    """Whole output of each compiled depthwise ring kernel (kernel size,
    stride, dtype, access width) against the reference; the stride-1 k3 and
    k5 16-byte kernels run three workgroups per CU with a 4-row ring."""
    _flush(f"dw_cl kernel: {_desc(wl)}")
    check_full(wl, force="dw_cl")


def _dw_generic_cases():
    """Channels-last depthwise calls for the generic dw_cl schedule: channel
    multipliers 1-4, kernels of any shape up to 9x9, strides 1-3, asymmetric
    padding, odd and even channel counts, every dtype, bias or not."""
    rng = np.random.default_rng(77)
    out = []
    i = 0
    while len(out) < 24:
        kh, kw = int(rng.integers(1, 10)), int(rng.integers(1, 10))
        sh, sw = int(rng.integers(1, 4)), int(rng.integers(1, 4))
        C = int(rng.choice([3, 8, 13, 64, 70]))
        m = int(rng.choice([1, 1, 2, 3, 4]))
        dtype = ["f32", "f16", "bf16"][i % 3]
        if dtype != "f32" and (C * m) % 2:
            C += 1
        H, W = int(rng.integers(kh, kh + 12)), int(rng.integers(kw, kw + 80))
        pb = [int(rng.integers(0, kh)), int(rng.integers(0, kw))]
        pa = [int(rng.integers(0, kh)), int(rng.integers(0, kw))]
        out.append(synth.random_case(7500 + i, rank=2, transposed=False, dtype=dtype, channels_last=True,
                                     N=int(rng.integers(1, 3)), C_in=C, C_out=C * m, groups=C, L=[H, W],
                                     k=[kh, kw], stride=[sh, sw], padding_before=pb, padding_after=pa,
                                     dilation=[1, 1], output_padding=[0, 0], has_bias=bool(i % 2)))
        i += 1
    return out


@pytest.mark.parametrize("wl", _dw_generic_cases(), ids=lambda v: v.name)
def test_dw_cl_generic_schedule(wl):
    """Whole output of the generic channels-last depthwise schedule (plan
    variant 2 of dw_cl, forced) against the reference."""
    _flush(f"dw_cl generic: {_desc(wl)}")
    check_full(wl, force="dw_cl", variant=2)


def _dw_mult_cases():
    """Multiplier 2 and 4 with even channel counts (the multiplier fan-out:
    one word load feeds 2m output channels), 16-bit, every compiled kernel
    width class (3 / 5 / 9) and column stride 1-3, ragged columns."""
    out = []
    i = 0
    for m in (2, 4):
        for kw, s in ((3, 1), (5, 2), (9, 3), (2, 1), (7, 2), (4, 3)):
            dtype = ("f16", "bf16")[i % 2]
            C = (16, 70)[i % 2]
            kh = (3, 1, 5)[i % 3]
            out.append(synth.random_case(7600 + i, rank=2, transposed=False, dtype=dtype, channels_last=True,
                                         N=2, C_in=C, C_out=C * m, groups=C, L=[kh + 6, 9 * s + kw + 13],
                                         k=[kh, kw], stride=[1 + i % 2, s], padding_before=[kh // 2, kw // 2],
                                         padding_after=[kh // 2, (kw - 1) // 2], dilation=[1, 1],
                                         output_padding=[0, 0], has_bias=bool(i % 2)))
            i += 1
    return out


@pytest.mark.parametrize("wl", _dw_mult_cases(), ids=lambda v: v.name)
def test_dw_cl_multiplier_fanout(wl):
    """Whole output of the generic schedule's multiplier fan-out kernels
    against the reference (the rule routes these calls to dw_cl variant 2)."""
    _flush(f"dw_cl multiplier: {_desc(wl)}")
    check_full(wl, force="dw_cl", variant=2)


def _dw1d_ncl_cases():
    """1-D depthwise calls on a channels-last (NLC) input, whose output is
    channel-major (NCL): multipliers 1-4, kernels 1-9, strides 1-3,
    asymmetric padding, output lengths that are and are not multiples of the
    8-output runs (so runs start on and off 16-byte boundaries), every dtype."""
    rng = np.random.default_rng(79)
    out = []
    for i in range(12):
        k = int(rng.integers(1, 10))
        s = int(rng.integers(1, 4))
        C = int(rng.choice([2, 8, 13, 64, 70]))
        m = int(rng.choice([1, 1, 2, 4]))
        dtype = ["f32", "f16", "bf16"][i % 3]
        if dtype != "f32" and (C * m) % 2:
            C += 1
        L = int(rng.integers(k, k + 300))
        pb, pa = int(rng.integers(0, k)), int(rng.integers(0, k))
        out.append(synth.random_case(7650 + i, rank=1, transposed=False, dtype=dtype, channels_last=True,
                                     N=int(rng.integers(1, 3)), C_in=C, C_out=C * m, groups=C, L=[L], k=[k],
                                     stride=[s], padding_before=[pb], padding_after=[pa], dilation=[1],
                                     output_padding=[0], has_bias=bool(i % 2)))
    return out


@pytest.mark.parametrize("wl", _dw1d_ncl_cases(), ids=lambda v: v.name)
def test_dw_cl_generic_1d_channel_major_output(wl):
    """Whole output of the generic channels-last schedule writing the NCL
    output of a 1-D call (per output channel, runs of 8 positions) against
    the reference, with the output strides the layout rule gives."""
    _flush(f"dw_cl generic, 1-D NCL output: {_desc(wl)}")
    y = check_full(wl, force="dw_cl", variant=2)
    assert y.stride(2) == 1 and y.stride(1) == y.shape[2]


def test_dw_cl_generic_schedule_exact_and_routed():
    """A multiplier-2 call routes to the generic schedule by the rule, and
    with wide integer inputs (outputs beyond 256, one rounding each) its
    bf16 result equals the reference rounded once."""
    import dataclasses
    wl = synth.random_case(7590, rank=2, transposed=False, dtype="bf16", channels_last=True, N=2, C_in=16, C_out=32,
                           groups=16, L=[12, 40], k=[5, 3], stride=[1, 2], padding_before=[2, 1],
                           padding_after=[2, 1], dilation=[1, 1], output_padding=[0, 0], has_bias=True)
    x, w, b = synth.make_inputs(wl)
    kw = expand_kw(wl)
    prep = api.Prepared(x, w, b, api.make_args(**{k: v for k, v in kw.items() if k not in ("groups", "transposed")},
                                               groups=wl.groups))
    assert api.kernel_name(prep.plan.kernel) == "dw_cl" and int(prep.plan.variant) == 2
    wl = dataclasses.replace(wl, x_dist=("ints", -127, 127), w_dist=("ints", -31, 31), b_dist=("ints", -500, 500))
    _flush(f"dw_cl generic exact: {_desc(wl)}")
    y = check_full(wl, exact=True)
    assert (y.abs().float() > 256).float().mean().item() > 0.2


# ------------------------------------- every grouped matrix-core kernel --

def _grp_mma_every_case():
    """One grouped 3x3 call per compiled matrix-core kernel: 4 or 8 channel
    slots (Cig 3 / 4 and 6 / 8), stride 1 and 2, fp16 / bf16, and planes of
    whole 16-byte chunks (position-major writes, HW % 8 == 0) or not."""
    out = []
    i = 0
    for pm in (True, False):
        for cp in (4, 8):
            for s in (1, 2):
                for dtype in ("f16", "bf16"):
                    cig = (3 if cp == 4 else 6) if pm else (4 if cp == 4 else 8)
                    if pm:
                        H, W, pa = (8, 12, 1) if s == 1 else (8, 16, 1)
                    else:
                        H, W, pa = (5, 12, 1) if s == 1 else (5, 14, 2)
                    cog = (8, 5)[i % 2]
                    out.append(synth.random_case(7400 + i, rank=2, transposed=False, dtype=dtype,
                                                 channels_last=False, N=3, C_in=2 * cig, C_out=2 * cog, groups=2,
                                                 L=[H, W], k=[3, 3], stride=[s, s], padding_before=[1, 1],
                                                 padding_after=[1, pa], dilation=[1, 1], output_padding=[0, 0],
                                                 has_bias=bool(i % 2)))
                    i += 1
    return out


@pytest.mark.parametrize("wl", _grp_mma_every_case(), ids=lambda v: v.name)
def test_grp_mma_every_kernel(wl):
    """Each compiled matrix-core grouped kernel (channel slots, stride, dtype,
    position-major or element-wise plane writes), checked to take that
    schedule, whole output against the reference."""
    _flush(f"grp matrix-core kernel: {_desc(wl)}")
    x, w, b = synth.make_inputs(wl, device="cuda")
    kw = expand_kw(wl)
    plan = api.Prepared(x, w, b, api.make_args(**{k: v for k, v in kw.items() if k not in ("groups", "transposed")},
                                               groups=wl.groups, transposed=wl.transposed),
                        force_kernel="grp").plan
    assert int(plan.variant) == 1, "shape chosen for the matrix-core schedule"
    check_full(wl, force="grp")


# ------------------- transposed 1-D, stride 2, both phases per workgroup --

def _t1_cases():
    """Transposed 1-D stride-2 calls inside the both-phases kernel's domain
    (16-bit, channel-contiguous x in whole 16-byte chunks): 2 to 8 taps,
    dilation 1 to 3 (an even dilation leaves one phase without taps),
    padding_before from 0 to 5, output_padding, groups, channel counts that are
    not multiples of the 32-channel block or the 64-channel tile, lengths below
    and above one 256-row tile, and both output layouts (contiguous, and
    channels-last through a channels-last weight)."""
    rng = np.random.default_rng(12)
    out = []
    i = 0
    while len(out) < 20:
        k = int(rng.integers(2, 9))
        dil = int(rng.choice([1, 1, 1, 2, 3]))
        pb = int(rng.integers(0, 6))
        pa = int(rng.integers(0, 6))
        op = int(rng.integers(0, max(2, dil)))
        L = int(rng.choice([5, 37, 256, 300, 777]))
        groups = int(rng.choice([1, 1, 2]))
        cig = int(rng.choice([8, 16, 40, 64, 104]))
        cog = int(rng.choice([1, 9, 64, 70, 130]))
        if (L - 1) * 2 - pb - pa + dil * (k - 1) + op + 1 < 1:
            continue
        wl = synth.random_case(7600 + i, rank=1, transposed=True, dtype=["bf16", "f16"][i % 2], channels_last=True,
                               N=int(rng.integers(1, 3)), C_in=groups * cig, C_out=groups * cog, groups=groups,
                               L=[L], k=[k], stride=[2], padding_before=[pb], padding_after=[pa], dilation=[dil],
                               output_padding=[op], has_bias=bool(i % 3))
        out.append((wl, i % 4 == 3))
        i += 1
    return out


def _t1_params():
    # Variant 12 on every case; variant 13 (eight waves) takes 2 or 4 taps.
    return [(wl, w_cl, v) for wl, w_cl in _t1_cases() for v in (12, 13) if v == 12 or wl.w_shape[2] in (2, 4)]


@pytest.mark.parametrize("wl,w_cl,variant", _t1_params(),
                         ids=lambda v: v.name if hasattr(v, "name") else str(v))
def test_transposed_both_phases_kernel(wl, w_cl, variant):
    """Whole output of the both-phases transposed kernels against the
    reference: plan variant 12 (four waves, two stages) and 13 (eight waves,
    three stages, 2 or 4 taps); w_cl stores the weight channels-last, which
    makes y channels-last too (channel-fastest write-out)."""
    _flush(f"transposed both phases, variant {variant} (w_cl={w_cl}): {_desc(wl)}")
    x, w, b = synth.make_inputs(wl, device="cuda")
    if w_cl:
        w = synth.channels_last_copy(w)
    kw = expand_kw(wl)
    prep = api.Prepared(x, w, b, api.make_args(**{k: v for k, v in kw.items() if k not in ("groups", "transposed")},
                                               groups=wl.groups, transposed=True),
                        force_kernel="igemm_t", force_variant=variant)
    assert api.kernel_name(prep.plan.kernel) == "igemm_t" and int(prep.plan.variant) == variant
    y = prep.run(x, w, b, prep.empty_output(x.device), prep.workspace(x.device))
    torch.cuda.synchronize()
    assert tuple(y.stride()) == oracle.out_strides(tuple(y.shape), tuple(x.shape), tuple(x.stride()),
                                                   tuple(w.shape), tuple(w.stride()))
    xr, wr, br = ref_inputs(x, w, b)
    yr, A = oracle.conv(xr, wr, br, **kw)
    assert_close(y, yr, A, EPS[wl.dtype], wl.name)


@pytest.mark.parametrize("offset", [0, 1, 3, 6])
@pytest.mark.parametrize("variant", [12, 13])
def test_both_phases_writes_stay_inside_output(variant, offset):
    """The both-phases kernels write contiguous output rows as 16-byte
    chunks aligned to y's memory, with the partial chunks at each row's ends
    element by element.  Here y (rows of the odd length 601, so every row
    starts at another alignment) sits at element offset `offset` inside a
    canary-filled buffer and starts as NaN: afterwards the canary is intact,
    no element is left NaN, and every element matches the reference (two
    row tiles, the second partial; two channel tiles, the second partial)."""
    wl = synth.random_case(7700 + offset, rank=1, transposed=True, dtype="bf16", channels_last=True, N=2, C_in=64,
                           C_out=70, groups=1, L=[301], k=[4], stride=[2], padding_before=[1], padding_after=[2],
                           dilation=[1], output_padding=[0], has_bias=True)
    _flush(f"both phases guard, variant {variant}, offset {offset}: {_desc(wl)}")
    x, w, b = synth.make_inputs(wl, device="cuda")
    kw = expand_kw(wl)
    prep = api.Prepared(x, w, b, api.make_args(**{k: v for k, v in kw.items() if k not in ("groups", "transposed")},
                                               groups=wl.groups, transposed=True),
                        force_kernel="igemm_t", force_variant=variant)
    assert tuple(prep.sizes) == (2, 70, 601) and tuple(prep.strides) == (70 * 601, 601, 1)
    span = 1 + sum((s - 1) * st for s, st in zip(prep.sizes, prep.strides))
    guard = 4096
    buf = torch.full((span + 2 * guard + 8,), 7.0, dtype=x.dtype, device="cuda")
    y = torch.as_strided(buf, prep.sizes, prep.strides, guard + offset)
    y.fill_(float("nan"))
    prep.run(x, w, b, y, prep.workspace(x.device))
    torch.cuda.synchronize()
    assert not torch.isnan(y).any()
    assert (buf[:guard + offset] == 7.0).all() and (buf[guard + offset + span:] == 7.0).all()
    xr, wr, br = ref_inputs(x, w, b)
    yr, A = oracle.conv(xr, wr, br, **kw)
    assert_close(y, yr, A, EPS[wl.dtype], wl.name)


def test_both_phases_plan_with_misaligned_x():
    """A both-phases plan whose x view starts off a 16-byte boundary (one
    element in): conv_run runs the call on the phase-split tile instead, with
    the same workspace, and the result is the reference's."""
    wl = synth.random_case(7710, rank=1, transposed=True, dtype="f16", channels_last=True, N=2, C_in=64, C_out=72,
                           groups=1, L=[300], k=[4], stride=[2], padding_before=[1], padding_after=[2], dilation=[1],
                           output_padding=[1], has_bias=True)
    _flush(f"both phases, misaligned x: {_desc(wl)}")
    x0, w, b = synth.make_inputs(wl, device="cuda")
    buf = torch.zeros(x0.numel() + 8, dtype=x0.dtype, device="cuda")
    x = torch.as_strided(buf, x0.shape, x0.stride(), 1)
    x.copy_(x0)
    kw = expand_kw(wl)
    prep = api.Prepared(x, w, b, api.make_args(**{k: v for k, v in kw.items() if k not in ("groups", "transposed")},
                                               groups=wl.groups, transposed=True))
    assert api.kernel_name(prep.plan.kernel) == "igemm_t" and int(prep.plan.variant) == 12
    y = prep.run(x, w, b, prep.empty_output(x.device), prep.workspace(x.device))
    torch.cuda.synchronize()
    xr, wr, br = ref_inputs(x0, w, b)
    yr, A = oracle.conv(xr, wr, br, **kw)
    assert_close(y, yr, A, EPS[wl.dtype], wl.name)


# ----------------------------------------------------- 1x1 plain GEMM --

def _one_cases():
    out = []
    shapes = [(2, [56, 56], 256, 256, "bf16"), (3, [30, 20], 128, 70, "f16"), (1, [1000], 64, 16, "bf16"),
              (2, [6, 7, 9], 192, 130, "f16"), (22, [56, 56], 256, 256, "bf16")]
    for i, (N, L, cin, cout, dt) in enumerate(shapes):
        r = len(L)
        out.append(synth.random_case(7700 + i, rank=r, transposed=False, dtype=dt, channels_last=True, N=N,
                                     C_in=cin, C_out=cout, groups=1, L=L, k=[1] * r, stride=[1] * r,
                                     padding_before=[0] * r, padding_after=[0] * r, dilation=[1] * r,
                                     output_padding=[0] * r, has_bias=bool(i % 2)))
    return out


@pytest.mark.parametrize("wl", _one_cases(), ids=lambda v: v.name)
def test_one_by_one_plain_gemm(wl):
    """1x1 calls on the plain-GEMM path (x's rows as A, the weight in place),
    whole output against the reference; the last case is large enough for
    the split-K rows past the last full round."""
    _flush(f"1x1: {_desc(wl)}")
    x, w, b = synth.make_inputs(wl, device="cuda")
    kw = expand_kw(wl)
    plan = api.Prepared(x, w, b, api.make_args(**{k: v for k, v in kw.items() if k not in ("groups", "transposed")},
                                               groups=1)).plan
    assert plan.flags & _abi.PLAN_ONE_BY_ONE
    if wl.x_shape[0] == 22:
        assert (int(plan.tile[7]) >> 24) > 1
    y = check_full(wl)
    # The same call with x at an odd element offset: the general gather
    # (no 16-byte loads) with the weight still read in place.
    buf = torch.zeros(x.numel() + 8, dtype=x.dtype, device="cuda")
    xm = torch.as_strided(buf, x.shape, x.stride(), 1)
    xm.copy_(x)
    ym = api.conv(xm, w, b)
    torch.cuda.synchronize()
    yr, A = oracle.conv(*ref_inputs(x, w, b))
    assert_close(ym, yr, A, EPS[wl.dtype], "1x1 misaligned x")


# ------------------------------------------- batches spanning 2 GiB --

@pytest.mark.parametrize("kind", ["dense", "depthwise"])
def test_batch_spanning_2gib(kind):
    """x and y of more than 2 GiB (bf16, channels-last): the plan runs the
    batch in chunks of images, each below the kernels' 32-bit buffer range.
    Whole images on both sides of the first chunk boundary and the last
    (smaller) chunk against the reference; the other images' outputs are
    finite (every chunk ran)."""
    g = torch.Generator(device="cuda").manual_seed(11)
    if kind == "dense":
        N, C, H, k = 600, 32, 256, 3
        w = (torch.randn((C, C, k, k), device="cuda", generator=g) / (C * k * k) ** 0.5).to(torch.bfloat16)
        groups = 1
    else:
        N, C, H, k = 400, 256, 112, 3
        w = (torch.randn((C, 1, k, k), device="cuda", generator=g) / k).to(torch.bfloat16)
        groups = C
    x = torch.empty_strided((N, C, H, H), (C * H * H, 1, H * C, C), dtype=torch.bfloat16, device="cuda")
    x.copy_(torch.randn((N, C, H, H), device="cuda", generator=g).to(torch.bfloat16))
    b = (0.1 * torch.randn((C,), device="cuda", generator=g)).to(torch.bfloat16)
    kw = dict(stride=(1, 1), padding_before=(1, 1), padding_after=(1, 1), dilation=(1, 1), groups=groups)
    prep = api.Prepared(x, w, b, api.make_args(**kw))
    nc = int(prep.plan.batch_chunk)
    _flush(f"2 GiB batch {kind}: N={N} chunk={nc} kernel={api.kernel_name(prep.plan.kernel)}")
    assert 0 < nc < N and N % nc
    y = prep.run(x, w, b, prep.empty_output(x.device), prep.workspace(x.device))
    torch.cuda.synchronize()
    assert bool(torch.isfinite(y.float().sum(dim=(1, 2, 3))).all())
    last = N - N % nc
    for n in sorted({0, nc - 1, nc, last - 1, last, N - 1}):
        xr, wr, br = ref_inputs(x[n:n + 1], w, b)
        yr, A = oracle.conv(xr, wr, br, **kw)
        assert_close(y[n:n + 1], yr, A, EPS["bf16"], f"{kind} image {n}")
    del x, y
    torch.cuda.empty_cache()


# ------------------------------------------- transposed depthwise (dw_cl) --

def _dwt_cases(n, seed):
    """Transposed depthwise calls inside the transposed generic schedule's
    domain: multiplier 1, dilation 1, kernels 1-9 (square or not), column
    stride 1 or 2, row stride 1-3, asymmetric padding, output_padding, 1-D
    and 2-D channels-last, every dtype, odd channel counts."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        i = len(out)
        r = 1 + int(rng.integers(0, 4) > 0)
        dtype = ["bf16", "f16", "f32"][i % 3]
        C = int(rng.choice([3, 16, 37, 64, 130]))
        k = [int(rng.integers(1, 10)) for _ in range(r)]
        s = [int(rng.integers(1, 4)) for _ in range(r - 1)] + [int(rng.integers(1, 3))]
        L = [int(rng.integers(2, 14)) for _ in range(r)]
        pb = [int(rng.integers(0, ki)) for ki in k]
        pa = [int(rng.integers(0, ki)) for ki in k]
        op = [int(rng.integers(0, si)) for si in s]
        if any((Li - 1) * si + ki + opi - pbi - pai < 1 for Li, si, ki, pbi, pai, opi in zip(L, s, k, pb, pa, op)):
            continue
        out.append(synth.random_case(9300 + i + 100 * seed, rank=r, transposed=True, dtype=dtype, channels_last=True,
                                     N=int(rng.integers(1, 3)), C_in=C, C_out=C, groups=C, L=L, k=k, stride=s,
                                     padding_before=pb, padding_after=pa, dilation=[1] * r, output_padding=op,
                                     has_bias=bool(rng.integers(0, 2))))
    return out


@pytest.mark.parametrize("wl", _dwt_cases(16, 1), ids=lambda v: v.name)
def test_transposed_depthwise_generic(wl):
    """Transposed depthwise calls on the dw_cl transposed schedule (the
    router's choice), whole output against the reference."""
    _flush(f"transposed depthwise: {_desc(wl)}")
    x, w, b = synth.make_inputs(wl, device="cuda")
    kw = expand_kw(wl)
    plan = api.Prepared(x, w, b, api.make_args(**{k: v for k, v in kw.items() if k not in ("groups", "transposed")},
                                               groups=wl.groups, transposed=wl.transposed)).plan
    assert api.kernel_name(plan.kernel) == "dw_cl" and int(plan.variant) == 2
    check_full(wl)
