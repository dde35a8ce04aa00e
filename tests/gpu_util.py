"""Helpers for the GPU parity tests: run the library, run the reference on the
same inputs, compare element by element within eps * A."""
import numpy as np
import torch

import oracle
from depthwise_stencil_implicit_amd import api, synth

# Per-element tolerance factor: |y_gpu - y| <= EPS * A + TINY, A = sum|x*w| + |b|.
EPS = {"f32": 1e-6, "f16": 2.0 ** -11, "bf16": 2.0 ** -8}
# The one rounding of the fp32 result into the output dtype errs by half an
# ulp; below the smallest normal number that is the absolute half-spacing of
# the subnormals, not a fraction of the value.
TINY = {torch.float32: 2.0 ** -150, torch.float16: 2.0 ** -25, torch.bfloat16: 2.0 ** -134}


def ref_inputs(x, w, b):
    f = lambda t: None if t is None else t.detach().double().cpu().contiguous().numpy()
    return f(x), f(w), f(b)


def expand_kw(wl):
    r = len(wl.x_shape) - 2
    ex = lambda v: tuple(v) * r if len(v) == 1 else tuple(v)
    return dict(stride=ex(wl.stride), padding_before=ex(wl.padding_before),
                padding_after=ex(wl.padding_after), dilation=ex(wl.dilation), groups=wl.groups,
                transposed=wl.transposed, output_padding=ex(wl.output_padding))


def run_gpu(wl, force=None, inputs=None, variant=None):
    x, w, b = inputs if inputs is not None else synth.make_inputs(wl, device="cuda")
    kw = expand_kw(wl)
    y = api.conv(x, w, b, stride=kw["stride"], padding_before=kw["padding_before"],
                 padding_after=kw["padding_after"], dilation=kw["dilation"], groups=kw["groups"],
                 transposed=kw["transposed"], output_padding=kw["output_padding"],
                 force_kernel=force, force_variant=variant)
    torch.cuda.synchronize()
    return x, w, b, y


def assert_close(y_gpu: torch.Tensor, y_ref: np.ndarray, A: np.ndarray, eps: float, what: str = ""):
    yg = y_gpu.detach().double().cpu().numpy()
    assert yg.shape == y_ref.shape, (yg.shape, y_ref.shape)
    err = np.abs(yg - y_ref)
    bad = ~(err <= eps * A + TINY[y_gpu.dtype])          # NaN counts as bad
    if bad.any():
        idx = np.argwhere(bad)[:5]
        detail = "; ".join(f"{tuple(i)}: gpu={yg[tuple(i)]!r} ref={y_ref[tuple(i)]!r} "
                           f"A={A[tuple(i)]!r}" for i in idx)
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outside eps*A ({eps}); {detail}")


def check_full(wl, force=None, exact=False, variant=None):
    """Whole output against the reference.  ``exact``: inputs whose fp32 sums
    are exact, so the result must equal the reference rounded once (nearest
    even) to the output dtype."""
    x, w, b, y = run_gpu(wl, force, variant=variant)
    xr, wr, br = ref_inputs(x, w, b)
    yr, A = oracle.conv(xr, wr, br, **expand_kw(wl))
    if exact:
        assert np.all(np.abs(yr) < 2.0 ** 24)
        rounded = torch.from_numpy(yr).to(torch.float32).to(y.dtype).double().numpy()
        yg = y.detach().double().cpu().numpy()
        bad = yg != rounded
        assert not bad.any(), f"{wl.name}: {int(bad.sum())} inexact, e.g. {yg[bad][:4]} vs {rounded[bad][:4]}"
    else:
        assert_close(y, yr, A, EPS[wl.dtype], wl.name)
    return y


def sample_points(shape, n, seed):
    """Random output indices plus every corner/edge combination."""
    rng = np.random.default_rng(seed)
    pts = [rng.integers(0, s, n) for s in shape]
    pts = np.stack(pts, axis=1)
    edges = []
    for combo in np.ndindex(*([3] * len(shape))):
        edges.append([0 if c == 0 else (s - 1 if c == 1 else s // 2) for c, s in zip(combo, shape)])
    return np.concatenate([pts, np.array(edges, dtype=np.int64)], axis=0)


def check_points(wl, n=4000, seed=0, force=None):
    """Sampled outputs against the reference, computed one by one."""
    x, w, b, y = run_gpu(wl, force)
    xr, wr, br = ref_inputs(x, w, b)
    pts = sample_points(tuple(y.shape), n, seed)
    yr, A = oracle.conv_points(xr, wr, br, pts, **expand_kw(wl))
    yg = y.detach()[tuple(torch.as_tensor(pts.T, device=y.device))].double().cpu().numpy()
    err = np.abs(yg - yr)
    bad = ~(err <= EPS[wl.dtype] * A + TINY[y.dtype])
    assert not bad.any(), f"{wl.name}: {int(bad.sum())} sampled outputs outside the bound, e.g. " \
                          f"{pts[bad][:3].tolist()} gpu={yg[bad][:3]} ref={yr[bad][:3]}"
    return y
