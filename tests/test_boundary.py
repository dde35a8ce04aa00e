"""Host logic of the boundary, on the CPU: binding rules and error contract,
output shapes and strides (against the reference's own, independently written
rule and torch), routing, forced kernels, and conv_run's checks."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from depthwise_stencil_implicit_amd import _abi as A
from depthwise_stencil_implicit_amd import api, synth


def T(shape, dtype=torch.bfloat16, cl=False):
    t = torch.empty(shape, dtype=dtype)
    return synth.channels_last_copy(t) if cl else t


def bind(x, w, b=None, **kw):
    return api.conv_bind(api.describe(x), api.describe(w), api.describe(b), api.make_args(**kw))


def bind_status(x, w, b=None, **kw):
    try:
        bind(x, w, b, **kw)
        return A.OK
    except api.ConvError as e:
        return e.status


def prep(x, w, b=None, force=None, **kw):
    return api.Prepared(x, w, b, api.make_args(**kw), force_kernel=force)


def wl_tensors(wl):
    x = T(wl.x_shape, synth.DTYPES[wl.dtype], wl.channels_last)
    w = T(wl.w_shape, synth.DTYPES[wl.dtype])
    c_out = wl.w_shape[1] * wl.groups if wl.transposed else wl.w_shape[0]
    b = T((c_out,), synth.DTYPES[wl.dtype]) if wl.has_bias else None
    return x, w, b


def wl_args(wl):
    r = len(wl.x_shape) - 2
    ex = lambda v: tuple(v) * r if len(v) == 1 else tuple(v)
    return dict(transposed=wl.transposed, groups=wl.groups, stride=ex(wl.stride),
                padding_before=ex(wl.padding_before), padding_after=ex(wl.padding_after),
                dilation=ex(wl.dilation), output_padding=ex(wl.output_padding) if wl.transposed else None)


# ------------------------------------------------------------------ binding --

def test_defaults_are_filled_and_broadcast():
    d = bind(T((2, 4, 9, 7)), T((6, 2, 3, 3)), groups=2, stride=2, padding_before=(1, 1), padding_after=(0, 2))
    assert d.spatial == 2 and d.N == 2 and d.C_in == 4 and d.C_out == 6 and d.groups == 2
    assert tuple(d.stride[:2]) == (2, 2) and tuple(d.dilation[:2]) == (1, 1)
    assert tuple(d.padding_before[:2]) == (1, 1) and tuple(d.padding_after[:2]) == (0, 2)
    assert tuple(d.out[:3]) == ((9 + 1 + 0 - 3) // 2 + 1, (7 + 1 + 2 - 3) // 2 + 1, 1)
    assert tuple(d.k[:3]) == (3, 3, 1) and d.has_bias == 0


def test_unbatched_input_gets_a_batch_dim():
    d = bind(T((4, 12)), T((8, 4, 3)), padding_before=1, padding_after=1)
    assert d.unbatched == 1 and d.N == 1 and d.x.rank == 3 and d.spatial == 1
    sizes, strides = api.conv_out_shape(d)
    assert sizes == (8, 12) and strides == (12, 1)


@pytest.mark.parametrize("k,dil,pb,pa", [(3, 1, 1, 1), (4, 1, 1, 2), (4, 2, 3, 3), (5, 3, 6, 6), (2, 1, 0, 1)])
def test_same_padding_split(k, dil, pb, pa):
    d = bind(T((1, 2, 11)), T((3, 2, k)), dilation=dil, padding_mode="same")
    assert (d.padding_before[0], d.padding_after[0], d.out[0]) == (pb, pa, 11)


def test_valid_padding():
    d = bind(T((1, 2, 11, 8)), T((3, 2, 3, 2)), padding_mode="valid")
    assert tuple(d.padding_before[:2]) == (0, 0) and tuple(d.out[:2]) == (9, 7)


@pytest.mark.parametrize("case", [
    dict(x=((1, 4, 8, 8), torch.float16), w=((4, 1, 3, 3), torch.bfloat16), kw=dict(groups=4)),  # dtype mismatch
    dict(x=((1, 4, 8, 8),), w=((4, 2, 3, 3),), kw=dict(groups=4)),            # Cig mismatch
    dict(x=((1, 6, 8, 8),), w=((4, 3, 3, 3),), kw=dict(groups=4)),            # C_in % groups
    dict(x=((1, 4, 8, 8),), w=((6, 1, 3, 3),), kw=dict(groups=4)),            # C_out % groups
    dict(x=((1, 4, 8, 8),), w=((4, 4, 3, 3),), kw=dict(padding_before=-1, padding_after=0)),
    dict(x=((1, 4, 8, 8),), w=((4, 4, 3, 3),), kw=dict(stride=0)),
    dict(x=((1, 4, 8, 8),), w=((4, 4, 3, 3),), kw=dict(dilation=0)),
    dict(x=((1, 4, 8, 8),), w=((4, 4, 3, 3),), kw=dict(groups=-1)),
    dict(x=((1, 4, 2, 2),), w=((4, 4, 3, 3),), kw=dict()),                    # output length < 1
    dict(x=((1, 4, 8, 8),), w=((4, 4, 3, 3),), kw=dict(stride=2, padding_mode="same")),
    dict(x=((1, 4, 8, 8),), w=((4, 4, 3, 3),), kw=dict(transposed=True, padding_mode="same")),
    dict(x=((1, 4, 8, 8),), w=((4, 4, 3, 3),), kw=dict(transposed=True, stride=2, output_padding=2)),
    dict(x=((1, 4, 8, 8),), w=((4, 4, 3, 3),), kw=dict(stride=2, output_padding=1)),  # forward op
    dict(x=((1, 4, 8, 8),), w=((4, 4, 3),), kw=dict()),                        # rank mismatch
    dict(x=((1, 4, 8, 8),), w=((4, 4),), kw=dict()),                           # weight rank < 3
    dict(x=((1, 4, 0, 8),), w=((4, 4, 3, 3),), kw=dict()),                     # empty spatial dim
    dict(x=((1, 4, 8, 8),), w=((4, 4, 3, 3),), kw=dict(stride=(1, 2, 3))),     # too many values
    dict(x=((1, 4, 8, 8),), w=((4, 4, 3, 3),), b=(5,), kw=dict()),            # bias size
])
def test_invalid_calls_are_rejected(case):
    x = T(*case["x"]) if len(case["x"]) == 2 else T(case["x"][0])
    w = T(*case["w"]) if len(case["w"]) == 2 else T(case["w"][0])
    b = T(case["b"]) if "b" in case else None
    assert bind_status(x, w, b, **case["kw"]) == A.EINVAL


def test_error_message_is_written():
    with pytest.raises(api.ConvError, match="divisible by groups"):
        bind(T((1, 6, 8, 8)), T((4, 3, 3, 3)), groups=4)


def test_aten_overload_mapping():
    """conv_transpose's symmetric padding p is a crop of p at each end; a
    'same' string maps to the padding mode; _convolution's flags are inert."""
    x, w = T((2, 4, 10)), T((4, 3, 3))
    d = bind(x, w, transposed=True, stride=2, padding_before=1, padding_after=1, output_padding=1)
    assert d.out[0] == (10 - 1) * 2 - 2 + 2 + 1 + 1 and d.C_out == 3
    d2 = bind(T((1, 3, 9, 9)), T((6, 3, 4, 4)), padding_mode="same")
    assert tuple(d2.padding_before[:2]) == (1, 1) and tuple(d2.padding_after[:2]) == (2, 2)


# ------------------------------------------------------------ shape/strides --

def _layout_cases():
    rng = np.random.default_rng(21)
    cases = []
    for i in range(60):
        r = int(rng.integers(1, 4))
        transposed = bool(rng.integers(0, 2))
        groups = int(rng.choice([1, 2, 4]))
        cig, cog = int(rng.integers(1, 4)), int(rng.integers(1, 4))
        L = [int(rng.integers(1, 9)) for _ in range(r)]
        k = [int(rng.integers(1, 4)) for _ in range(r)]
        s = [int(rng.integers(1, 4)) for _ in range(r)]
        d = [int(rng.integers(1, 3)) for _ in range(r)]
        pb = [int(rng.integers(0, 3)) for _ in range(r)]
        pa = [int(rng.integers(0, 3)) for _ in range(r)]
        op = [int(rng.integers(0, max(a, b))) if transposed else 0 for a, b in zip(s, d)]
        N = int(rng.choice([0, 1, 3]))
        cl = bool(rng.integers(0, 2))
        wcl = bool(rng.integers(0, 4) == 0)
        cases.append((r, transposed, groups, cig, cog, L, k, s, d, pb, pa, op, N, cl, wcl))
    return cases


@pytest.mark.parametrize("case", _layout_cases())
def test_out_shape_and_strides_match_reference_rule(case):
    r, transposed, groups, cig, cog, L, k, s, d, pb, pa, op, N, cl, wcl = case
    x = T((N, groups * cig) + tuple(L), cl=cl)
    w = T(((groups * cig, cog) if transposed else (groups * cog, cig)) + tuple(k), cl=wcl)
    kw = dict(transposed=transposed, groups=groups, stride=s, padding_before=pb, padding_after=pa, dilation=d,
              output_padding=op if transposed else None)
    ref_shape = oracle.out_shape(tuple(x.shape), tuple(w.shape), stride=s, padding_before=pb,
                                 padding_after=pa, dilation=d, groups=groups, transposed=transposed,
                                 output_padding=op)
    if any(o < 1 for o in ref_shape[2:]):
        assert bind_status(x, w, **kw) == A.EINVAL
        return
    dd = bind(x, w, **kw)
    sizes, strides = api.conv_out_shape(dd)
    assert sizes == ref_shape
    assert strides == oracle.out_strides(ref_shape, tuple(x.shape), tuple(x.stride()), tuple(w.shape),
                                         tuple(w.stride()))


EXPECTED = {  # (sizes, strides, kernel) of the five workloads
    "dw_f32_nchw_1x32x32x32_k3": ((1, 32, 32, 32), (32768, 1024, 32, 1), "plane"),
    "dw_bf16_nhwc_32x256x56x56_k3s1": ((32, 256, 56, 56), (802816, 1, 14336, 256), "dw_cl"),
    "dw_bf16_nhwc_32x256x56x56_k5s1": ((32, 256, 56, 56), (802816, 1, 14336, 256), "dw_cl"),
    "dw_bf16_nhwc_32x256x56x56_k7s1": ((32, 256, 56, 56), (802816, 1, 14336, 256), "dw_cl"),
    "dw_bf16_nhwc_32x256x56x56_k3s2": ((32, 256, 28, 28), (200704, 1, 7168, 256), "dw_cl"),
    "dw_bf16_nhwc_32x256x56x56_k5s2": ((32, 256, 28, 28), (200704, 1, 7168, 256), "dw_cl"),
    "dw_bf16_nhwc_32x256x56x56_k7s2": ((32, 256, 28, 28), (200704, 1, 7168, 256), "dw_cl"),
    "grp_f16_nchw_32x256x28x28_g64_m2": ((32, 512, 28, 28), (401408, 784, 28, 1), ("grp", "plane")),
    "dense_bf16_nhwc_64x256x56x56_k3": ((64, 256, 56, 56), (802816, 1, 14336, 256), "igemm"),
    "convT1d_bf16_nlc_16x512x8192_k4s2": ((16, 512, 16383), (8388096, 16383, 1), "igemm_t"),
}


@pytest.mark.parametrize("wl", synth.all_workloads(), ids=lambda w: w.name)
def test_workload_layouts_and_routes(wl):
    x, w, b = wl_tensors(wl)
    p = prep(x, w, b, **wl_args(wl))
    sizes, strides, kern = EXPECTED[wl.name]
    assert p.sizes == sizes and p.strides == strides
    kern = kern if isinstance(kern, tuple) else (kern,)
    assert api.kernel_name(p.plan.kernel) in kern


def test_workload_algorithmic_counts():
    got = {}
    for wl in synth.all_workloads():
        x, w, b = wl_tensors(wl)
        p = prep(x, w, b, **wl_args(wl))
        got[wl.name] = (p.plan.flops, p.plan.bytes)
    assert got["dense_bf16_nhwc_64x256x56x56_k3"] == (2 * 200704 * 256 * 2304, 206701056)
    # transposed: 2 taps of parity per output, 16383 outputs per (n, co, ci)
    assert got["convT1d_bf16_nlc_16x512x8192_k4s2"] == (2 * 16 * 512 * 512 * 32766, 404733952)
    assert got["grp_f16_nchw_32x256x28x28_g64_m2"] == (2 * 32 * 512 * 784 * 36, 38572032)
    assert got["dw_bf16_nhwc_32x256x56x56_k7s1"] == (2 * 32 * 256 * 3136 * 49, 102786048)
    assert got["dw_f32_nchw_1x32x32x32_k3"] == (589824, 263424)


# -------------------------------------------------- plan / failure contract --

def test_forced_kernel_outside_its_domain_is_refused():
    x, w = T((2, 8, 12, 12)), T((8, 1, 3, 3))
    kw = dict(groups=8, padding_before=1, padding_after=1)
    with pytest.raises(api.ConvError) as e:
        prep(x, w, force="dw_cl", **kw)          # NCHW input: no channel-contiguous schedule
    assert e.value.status == A.EUNSUPPORTED
    with pytest.raises(api.ConvError) as e:
        prep(x, w, force="igemm_t", **kw)        # forward call on the transposed kernel
    assert e.value.status == A.EUNSUPPORTED
    with pytest.raises(api.ConvError) as e:
        prep(T((1, 18, 8, 8)), T((4, 9, 3, 3)), force="plane", groups=2)   # 9 channels per group
    assert e.value.status == A.EUNSUPPORTED
    for k in ("plane", "reduce", "igemm"):
        prep(x, w, force=k, **kw)                # inside their domains


def test_output_layout_mismatch_is_refused():
    x, w = T((2, 8, 12, 12)), T((8, 1, 3, 3))
    d = bind(x, w, groups=8, padding_before=1, padding_after=1)
    sizes, strides = api.conv_out_shape(d)
    good = api.tensor_desc(sizes, strides, torch.bfloat16)
    api.conv_plan(d, good)
    for bad_sizes, bad_strides in [(sizes, (strides[0], 1, strides[2] * 8, 8)),
                                   ((2, 8, 12, 11), strides)]:
        with pytest.raises(api.ConvError) as e:
            api.conv_plan(d, api.tensor_desc(bad_sizes, bad_strides, torch.bfloat16))
        assert e.value.status == A.ELAYOUT
    with pytest.raises(api.ConvError) as e:
        api.conv_plan(d, api.tensor_desc(sizes, strides, torch.float16))
    assert e.value.status == A.ELAYOUT


def test_routing_rules():
    name = lambda p: api.kernel_name(p.plan.kernel)
    # depthwise channels-last with a compiled schedule -> dw_cl; same call NCHW -> plane
    assert name(prep(T((1, 16, 9, 9), cl=True), T((16, 1, 3, 3)), groups=16)) == "dw_cl"
    assert name(prep(T((1, 16, 9, 9)), T((16, 1, 3, 3)), groups=16)) == "plane"
    # dilation, 3-D, wide groups, dense -> igemm
    assert name(prep(T((1, 16, 9, 9)), T((16, 1, 3, 3)), groups=16, dilation=2)) == "igemm"
    assert name(prep(T((1, 16, 5, 5, 5)), T((16, 1, 3, 3, 3)), groups=16)) == "igemm"
    assert name(prep(T((1, 32, 9, 9)), T((32, 16, 3, 3)), groups=2)) == "igemm"
    assert name(prep(T((1, 8, 9, 9)), T((8, 8, 3, 3)))) == "igemm"
    # a large kernel over a tiny input -> reduce
    assert name(prep(T((1, 16, 7, 7)), T((16, 1, 7, 7)), groups=16)) == "reduce"
    # 1-D depthwise runs on the stencil with H = 1
    assert name(prep(T((2, 16, 40)), T((16, 1, 5)), groups=16)) == "plane"
    # every transposed call -> igemm_t
    assert name(prep(T((1, 8, 9)), T((8, 4, 3)), transposed=True, groups=2)) == "igemm_t"


def test_plans_are_deterministic():
    x, w, b = T((4, 64, 20, 20), cl=True), T((64, 64, 3, 3)), T((64,))
    p1 = prep(x, w, b, padding_before=1, padding_after=1).plan
    p2 = prep(x, w, b, padding_before=1, padding_after=1).plan
    assert bytes(p1) == bytes(p2)


def test_run_checks_before_touching_the_device():
    x, w = T((2, 8, 12, 12), cl=True), T((8, 8, 3, 3))
    p = prep(x, w, None, padding_before=1, padding_after=1)
    assert p.plan.workspace_bytes > 0
    L = A.lib()
    run = lambda *a: L.conv_run(ctypes.byref(p.plan), *a)
    assert run(0x1001, 0x2000, None, 0x3000, 0x4000, p.plan.workspace_bytes, None) == A.EALIGN
    assert run(None, 0x2000, None, 0x3000, 0x4000, p.plan.workspace_bytes, None) == A.EINVAL
    assert run(0x1000, 0x2000, 0x5000, 0x3000, 0x4000, p.plan.workspace_bytes, None) == A.EINVAL  # bias
    assert run(0x1000, 0x2000, None, 0x3000, None, 0, None) == A.EINVAL                            # workspace
    assert run(0x1000, 0x2000, None, 0x3000, 0x4000, p.plan.workspace_bytes - 1, None) == A.EINVAL
    if not torch.cuda.is_available():
        assert run(0x1000, 0x2000, None, 0x3000, 0x4000, p.plan.workspace_bytes, None) == A.EDEVICE


def test_empty_output_runs_as_a_noop_without_a_device():
    x, w = T((0, 8, 12, 12)), T((8, 1, 3, 3))
    p = prep(x, w, groups=8)
    assert p.plan.grid[0] == 0
    assert A.lib().conv_run(ctypes.byref(p.plan), None, None, None, None, None, 0, None) == A.OK


def test_cpu_tensors_are_refused_by_the_product_path():
    with pytest.raises(ValueError, match="GPU only"):
        api.conv(torch.zeros((1, 2, 5)), torch.zeros((2, 2, 3)))


# ------------------------------------------- explicit schedules, LDS budget --

def test_wide_grouped_product_goes_to_the_gemm():
    """A grouped call with few input channels per group but a wide per-group
    output: the grouped stencil keeps every group's weights in LDS, which do
    not fit, so the planner picks the implicit GEMM, and forcing the grouped
    kernel is refused."""
    x, w = T((1, 16, 32, 32), torch.float16), T((2048, 8, 9, 9), torch.float16)
    p = prep(x, w, groups=2, padding_before=4, padding_after=4).plan
    assert api.kernel_name(p.kernel) == "igemm" and p.lds_bytes <= 160 * 1024
    with pytest.raises(api.ConvError) as e:
        prep(x, w, groups=2, padding_before=4, padding_after=4, force="grp")
    assert e.value.status == A.EUNSUPPORTED
    x2, w2 = T((1, 16, 32, 32), torch.float16), T((1024, 8, 3, 3), torch.float16)
    p2 = prep(x2, w2, groups=2, padding_before=1, padding_after=1).plan
    assert api.kernel_name(p2.kernel) == "igemm"
    # A narrow per-group output still runs on the grouped stencil.
    p3 = prep(T((1, 16, 32, 32), torch.float16), T((32, 8, 3, 3), torch.float16), groups=2,
              padding_before=1, padding_after=1).plan
    assert api.kernel_name(p3.kernel) == "grp" and p3.lds_bytes <= 64 * 1024


def test_forced_schedule_is_explicit():
    """conv_plan_ex takes the implicit GEMM's tile index and the grouped
    kernel's schedule; a schedule of the wrong dtype class is refused, a
    schedule without a kernel is invalid, and the environment plays no part."""
    import os
    x, w = T((2, 64, 12, 12), cl=True), T((64, 64, 3, 3))
    for v in (0, 3, 9, 11):
        p = api.Prepared(x, w, None, api.make_args(padding_before=1, padding_after=1), force_kernel="igemm",
                         force_variant=v).plan
        assert p.variant == v
    with pytest.raises(api.ConvError) as e:
        api.Prepared(x, w, None, api.make_args(padding_before=1, padding_after=1), force_kernel="igemm",
                     force_variant=5)       # the fp32 tile
    assert e.value.status == A.EUNSUPPORTED
    with pytest.raises(api.ConvError) as e:
        api.Prepared(x, w, None, api.make_args(padding_before=1, padding_after=1), force_variant=0)
    assert e.value.status == A.EINVAL
    base = bytes(prep(x, w, padding_before=1, padding_after=1).plan)
    old = os.environ.get("MICONV_IGEMM_CFG")
    os.environ["MICONV_IGEMM_CFG"] = "4"
    try:
        assert bytes(prep(x, w, padding_before=1, padding_after=1).plan) == base
    finally:
        if old is None:
            del os.environ["MICONV_IGEMM_CFG"]
        else:
            os.environ["MICONV_IGEMM_CFG"] = old
    # The grouped kernel: the matrix-core schedule only where it applies.
    xg, wg = T((2, 8, 8, 16), torch.float16), T((16, 4, 3, 3), torch.float16)
    pg = api.Prepared(xg, wg, None, api.make_args(groups=2, padding_before=1, padding_after=1),
                      force_kernel="grp").plan
    assert pg.variant == 1
    pv = api.Prepared(xg, wg, None, api.make_args(groups=2, padding_before=1, padding_after=1),
                      force_kernel="grp", force_variant=0).plan
    assert pv.variant == 0
    with pytest.raises(api.ConvError):
        api.Prepared(T((2, 8, 8, 15), torch.float16), wg, None,
                     api.make_args(groups=2, padding_before=1, padding_after=1), force_kernel="grp",
                     force_variant=1)


# -------------------------------------------------------------- gradients --

def _bwd(wl, gy_strides=None):
    x, w, b = wl_tensors(wl)
    p = prep(x, w, b, **wl_args(wl))
    gy = torch.empty_strided(p.sizes, gy_strides or p.strides, dtype=x.dtype)
    return x, w, api.PreparedBackward(x, w, gy, api.make_args(**wl_args(wl)))


def test_gradient_layouts_of_the_workloads():
    """dx has the layout of the adjoint call's output (channels-last for the
    channels-last 2-D calls, contiguous for the 1-D transposed call whose gy
    is contiguous), dw is dense in w's format, db is [C_out]."""
    want = {"dense_bf16_nhwc_64x256x56x56_k3": (802816, 1, 14336, 256),
            "convT1d_bf16_nlc_16x512x8192_k4s2": (4194304, 8192, 1),
            "grp_f16_nchw_32x256x28x28_g64_m2": (200704, 784, 28, 1),
            "dw_bf16_nhwc_32x256x56x56_k7s2": (802816, 1, 14336, 256)}
    for wl in synth.all_workloads():
        x, w, bp = _bwd(wl)
        assert bp.dx_layout[0] == tuple(x.shape)
        if wl.name in want:
            assert bp.dx_layout[1] == want[wl.name], wl.name
        assert bp.dw_layout == (tuple(w.shape), tuple(w.stride()))
        c_out = wl.w_shape[1] * wl.groups if wl.transposed else wl.w_shape[0]
        assert bp.db_layout == ((c_out,), (1,))


def test_gradient_schedules():
    """The dense call's weight gradient runs on the matrix cores with both
    operands channel-major; the transposed 1-D call's contiguous gy is first
    copied channels-last (wg_tile[6] bytes), so both of its gradients read
    channel-major operands too; channels-last 16-bit depthwise weight gradients use
    the depthwise stencil (mode 8), channel-major few-channel ones (fp32
    depthwise NCHW, the grouped workload) the plane-staged schedule (16); the
    input gradient of a forward call is a transposed call and vice versa,
    except stride-1 stencil calls, whose dx is a forward call on the reversed
    weight."""
    _, _, dense = _bwd(synth.dense_bf16_cl())
    assert dense.plan.wg_tile[0] == 1 and api.kernel_name(dense.plan.dgrad.kernel) == "igemm_t"
    _, _, tr = _bwd(synth.transposed_bf16_nlc())
    assert tr.plan.wg_tile[0] == 1 and api.kernel_name(tr.plan.dgrad.kernel) == "igemm"
    assert tr.plan.wg_tile[6] == 16 * 512 * 16383 * 2 and tr.plan.workspace_bytes > tr.plan.wg_tile[6]
    _, _, dw = _bwd(synth.depthwise_bf16_cl(3, 1))
    assert dw.plan.wg_tile[0] == 8 and dw.plan.dgrad_flip == 1 and api.kernel_name(dw.plan.dgrad.kernel) == "dw_cl"
    _, _, dw2 = _bwd(synth.depthwise_bf16_cl(5, 2))
    assert dw2.plan.wg_tile[0] == 8 and dw2.plan.dgrad_flip == 0
    _, _, small = _bwd(synth.depthwise_f32_small())
    assert small.plan.wg_tile[0] == 16 and small.plan.dgrad_flip == 1
    _, _, gp = _bwd(synth.grouped_f16())
    assert gp.plan.wg_tile[0] == 16 and gp.plan.dgrad_flip == 1 and api.kernel_name(gp.plan.dgrad.kernel) == "grp"
    assert dense.plan.flops[1] == dense.plan.flops[0] == 2 * 200704 * 256 * 2304
    assert dense.plan.workspace_bytes >= dense.plan.wg_tile[3] * 9 * 256 * 256 * 4


def test_gradient_plan_errors():
    x, w = T((1, 4, 9)), T((4, 2, 3))
    # A transposed call whose output_padding reaches the stride: its forward
    # adjoint would be longer than x.
    a = api.make_args(transposed=True, stride=2, dilation=3, output_padding=2, padding_before=0, padding_after=0)
    d = api.conv_bind(api.describe(x), api.describe(w), None, a)
    sizes, strides = api.conv_out_shape(d)
    gy = api.tensor_desc(sizes, strides, torch.bfloat16)
    p = A.ConvBwdPlan()
    assert A.lib().conv_plan_backward(ctypes.byref(d), ctypes.byref(gy), 1, 0, 0, ctypes.byref(p)) == A.EUNSUPPORTED
    # ... though its weight and bias gradients can be planned.
    assert A.lib().conv_plan_backward(ctypes.byref(d), ctypes.byref(gy), 0, 1, 1, ctypes.byref(p)) == A.OK
    # gy of the wrong shape.
    bad = api.tensor_desc((1, 2, sizes[2] + 1), (sizes[2] + 1, 1, 1), torch.bfloat16)
    assert A.lib().conv_plan_backward(ctypes.byref(d), ctypes.byref(bad), 1, 1, 1, ctypes.byref(p)) == A.ELAYOUT


def test_gradient_run_checks_before_touching_the_device():
    x, w, bp = _bwd(synth.dense_bf16_cl().with_batch(1))
    L = A.lib()
    run = lambda *a: L.conv_run_backward(ctypes.byref(bp.plan), *a)
    ws = bp.plan.workspace_bytes
    assert run(0x1000, 0x2000, None, 0x3000, 0x4000, 0x5000, 0x6000, ws, None) == A.EINVAL        # no gy
    assert run(0x1000, None, 0x2000, 0x3000, 0x4000, 0x5000, 0x6000, ws, None) == A.EINVAL        # dx needs w
    assert run(0x1000, 0x2000, 0x2200, 0x3000, 0x4000, 0x5000, None, 0, None) == A.EINVAL         # workspace
    assert run(0x1001, 0x2000, 0x2200, 0x3000, 0x4000, 0x5000, 0x6000, ws, None) == A.EALIGN


# ------------------------------------------------------------ 1x1 calls --

def test_one_by_one_plain_gemm_plan():
    """A forward 1x1 call with stride 1 and no padding on dense
    channels-last x, with a contiguous weight and C_in a multiple of 64, is a
    plain GEMM: the plan flags it and needs no weight workspace."""
    x, w, b = T((4, 256, 28, 28), cl=True), T((384, 256, 1, 1)), T((384,))
    p = prep(x, w, b).plan
    assert p.flags & A.PLAN_ONE_BY_ONE and api.kernel_name(p.kernel) == "igemm"
    assert p.workspace_bytes == 0 or (p.tile[7] >> 24) > 1      # only split-K partial sums, if any
    p1 = prep(T((2, 128, 50), cl=True), T((64, 128, 1))).plan
    assert p1.flags & A.PLAN_ONE_BY_ONE
    # Not a plain GEMM: NCHW x, padding, stride, C_in not a multiple of 64,
    # transposed, grouped.
    assert not prep(T((4, 256, 28, 28)), w).plan.flags
    assert not prep(x, w, padding_before=1, padding_after=1).plan.flags
    assert not prep(x, w, stride=2).plan.flags
    assert not prep(T((4, 96, 28, 28), cl=True), T((64, 96, 1, 1))).plan.flags
    assert not prep(T((4, 256, 28, 28), cl=True), T((256, 64, 1, 1)), transposed=True).plan.flags
    assert not prep(x, T((384, 128, 1, 1)), groups=2).plan.flags


# ------------------------------------------------------ schedule timing --

def _cands(wl):
    x, w, b = wl_tensors(wl)
    p = prep(x, w, b, **wl_args(wl))
    return p, api.conv_plan_candidates(p.desc, api.tensor_desc(p.sizes, p.strides, x.dtype))


def test_candidates_cover_every_schedule():
    """The rule's plan comes first; the dense call lists every 16-bit tile
    configuration; the transposed 1-D call adds the both-phases kernels; the
    depthwise call lists the ring stencil and the plane stencil but not the
    implicit GEMM, whose one input channel per group would be padded to a
    64-channel block; each candidate is a plan conv_plan_ex accepts, listed
    once."""
    p, c = _cands(synth.dense_bf16_cl())
    assert bytes(c[0]) == bytes(p.plan)
    assert sorted({int(q.variant) for q in c if api.kernel_name(q.kernel) == "igemm"}) == [0, 1, 2, 3, 4, 6, 7, 8, 9, 10]
    _, c = _cands(synth.transposed_bf16_nlc())
    assert {12, 13} <= {int(q.variant) for q in c}
    _, c = _cands(synth.depthwise_bf16_cl(5, 1))
    assert {"dw_cl", "plane"} <= {api.kernel_name(q.kernel) for q in c}
    assert not {"reduce", "igemm"} & {api.kernel_name(q.kernel) for q in c}
    keys = [(q.kernel, q.variant, q.flags) for q in c]
    assert len(keys) == len(set(keys))
    _, c = _cands(synth.grouped_f16())
    assert {(api.kernel_name(q.kernel), int(q.variant)) for q in c} >= {("grp", 0), ("grp", 1), ("plane", 0)}


def test_untuned_call_plans_by_the_rule():
    p, _ = _cands(synth.dense_bf16_cl())
    t = api.conv_plan_tuned(p.desc, api.tensor_desc(p.sizes, p.strides, torch.bfloat16))
    assert not (t.flags & A.PLAN_TUNED) and bytes(t) == bytes(p.plan)


def test_batch_spanning_2gib_runs_in_chunks():
    """x (or y) spanning 2 GiB or more: the kernels take 32-bit buffer
    offsets, so the plan covers a chunk of images whose spans stay below
    2 GiB; d and y stay the whole call (FLOPs and bytes of the whole call),
    and the workspace also covers the last, smaller chunk."""
    N, C, H = 600, 32, 256
    x = torch.empty_strided((N, C, H, H), (C * H * H, 1, H * C, C), dtype=torch.bfloat16)   # NHWC, not touched
    w = T((C, C, 3, 3))
    p = prep(x, w, padding_before=1, padding_after=1)
    nc = int(p.plan.batch_chunk)
    assert 0 < nc < N and N % nc
    assert int(p.plan.d.N) == N and int(p.plan.y.sizes[0]) == N and tuple(p.sizes)[0] == N
    img = C * H * H * 2
    assert nc * img <= (1 << 31) - 4096 < (nc + 1) * img
    assert api.kernel_name(p.plan.kernel) == "igemm"
    assert int(p.plan.flops) == 2 * N * H * H * C * C * 9
    # A batch that fits is one launch.
    small = torch.empty_strided((8, C, H, H), (C * H * H, 1, H * C, C), dtype=torch.bfloat16)
    assert int(prep(small, w, padding_before=1, padding_after=1).plan.batch_chunk) == 0


def test_dw1d_channels_last_input_routes_to_generic_dw_cl():
    """A 1-D depthwise call on an NLC input has a channel-major (NCL) output by
    the layout rule; the planner sends it to the generic channels-last
    schedule, which writes runs of positions per channel."""
    wl = next(w for w in synth.domain_edge_workloads() if w.name.startswith("edge_dw1d"))
    x, w, b = wl_tensors(wl)
    p = prep(x, w, b, **wl_args(wl))
    assert p.strides[2] == 1 and p.strides[1] == p.sizes[2]
    assert api.kernel_name(p.plan.kernel) == "dw_cl" and int(p.plan.variant) == 2


def test_generic_depthwise_candidate_only_without_a_ring_schedule():
    """Where a ring schedule applies (3x3 stride 2) the candidates leave out
    the generic channels-last schedule, which times well only on warm
    buffers; a multiplier-2 call (no ring schedule) keeps it."""
    _, c = _cands(synth.depthwise_bf16_cl(3, 2))
    dw = {int(q.variant) for q in c if api.kernel_name(q.kernel) == "dw_cl"}
    assert 2 not in dw and dw
    m2 = next(w for w in synth.domain_edge_workloads() if w.name.endswith("_m2"))
    _, c = _cands(m2)
    assert 2 in {int(q.variant) for q in c if api.kernel_name(q.kernel) == "dw_cl"}
