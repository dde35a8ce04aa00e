"""Pins for the double-precision reference convolution (``oracle/``).

The reference is checked here against things other than itself: hand-derived
worked examples of the pages' index maps (tests/golden), torch's CPU float64
convolution routines, closed forms (delta and all-ones kernels), the adjoint
identity, an exhaustive operator-matrix transpose check, the textbook rewrite
of a transposed convolution as a zero-inserted, kernel-flipped forward one,
the 1x1-conv-is-a-matmul identity, and the group decomposition.  Each is
chosen so that a dropped term, a wrong sign or index, or swapped weight axes
fail at least one test.
"""
import glob
import json
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from depthwise_stencil_implicit_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
CONV = {1: F.conv1d, 2: F.conv2d, 3: F.conv3d}
CONVT = {1: F.conv_transpose1d, 2: F.conv_transpose2d, 3: F.conv_transpose3d}


def torch_ref(x, w, b, *, stride, padding_before, padding_after, dilation, groups, transposed,
              output_padding):
    """torch CPU float64 convolution, with asymmetric padding expressed by an
    explicit pad (forward) or a crop of the uncropped output (transposed)."""
    x = torch.as_tensor(np.asarray(x, dtype=np.float64))
    w = torch.as_tensor(np.asarray(w, dtype=np.float64))
    r = x.dim() - 2
    if not transposed:
        pads = []
        for i in reversed(range(r)):
            pads += [padding_before[i], padding_after[i]]
        y = CONV[r](F.pad(x, pads), w, None, stride=tuple(stride), padding=0,
                    dilation=tuple(dilation), groups=groups)
    else:
        full = CONVT[r](x, w, None, stride=tuple(stride), padding=0, output_padding=0,
                        groups=groups, dilation=tuple(dilation))
        ext = []
        for i in reversed(range(r)):
            ext += [0, output_padding[i]]
        full = F.pad(full, ext)
        sl = [slice(None), slice(None)]
        for i in range(r):
            L_full = full.shape[2 + i] - output_padding[i]
            sl.append(slice(padding_before[i], L_full - padding_after[i] + output_padding[i]))
        y = full[tuple(sl)]
    if b is not None:
        bb = torch.as_tensor(np.asarray(b, dtype=np.float64))
        y = y + bb.reshape((1, -1) + (1,) * r)
    return y.numpy()


def kw_of(wl):
    r = len(wl.x_shape) - 2
    ex = lambda v: tuple(v) * r if len(v) == 1 else tuple(v)
    return dict(stride=ex(wl.stride), padding_before=ex(wl.padding_before),
                padding_after=ex(wl.padding_after), dilation=ex(wl.dilation), groups=wl.groups,
                transposed=wl.transposed, output_padding=ex(wl.output_padding))


def as64(t):
    return None if t is None else t.double().contiguous().numpy()


# --------------------------------------------------------------- golden --

@pytest.mark.parametrize("path", sorted(glob.glob(os.path.join(GOLDEN, "*.json"))),
                         ids=lambda p: os.path.basename(p))
def test_golden_fixture(oracle_mod, path):
    with open(path) as f:
        fx = json.load(f)
    op = fx["op"]
    y, A = oracle_mod.conv(np.array(fx["x"], float), np.array(fx["w"], float),
                           None if fx["b"] is None else np.array(fx["b"], float),
                           stride=op["stride"], padding_before=op["padding_before"],
                           padding_after=op["padding_after"], dilation=op["dilation"],
                           groups=op["groups"], transposed=op["transposed"],
                           output_padding=op["output_padding"])
    np.testing.assert_array_equal(y, np.array(fx["y"], float))
    assert (A >= np.abs(y)).all()


# ------------------------------------------------------ library routine --

def _cases():
    rng = np.random.default_rng(7)
    cases = []
    seed = 100
    for rank in (1, 2, 3):
        for transposed in (False, True):
            for _ in range(6 if rank < 3 else 3):
                seed += 1
                groups = int(rng.choice([1, 2, 3]))
                cig = int(rng.integers(1, 4))
                cog = int(rng.integers(1, 4))
                L = [int(rng.integers(3, 9 if rank < 3 else 6)) for _ in range(rank)]
                k = [int(rng.integers(1, 4)) for _ in range(rank)]
                s = [int(rng.integers(1, 4)) for _ in range(rank)]
                d = [int(rng.integers(1, 3)) for _ in range(rank)]
                pb = [int(rng.integers(0, 3)) for _ in range(rank)]
                pa = [int(rng.integers(0, 3)) for _ in range(rank)]
                op = [int(rng.integers(0, max(si, di))) if transposed else 0
                      for si, di in zip(s, d)]
                if transposed:   # keep the crop inside the uncropped output
                    ok = all((Li - 1) * si + di * (ki - 1) + 1 + opi - pbi - pai >= 1
                             for Li, si, di, ki, pbi, pai, opi in zip(L, s, d, k, pb, pa, op))
                else:
                    ok = all(Li + pbi + pai - di * (ki - 1) - 1 >= 0
                             for Li, pbi, pai, di, ki in zip(L, pb, pa, d, k))
                if not ok:
                    continue
                cases.append(synth.random_case(
                    seed, rank=rank, transposed=transposed, dtype="f32", channels_last=False,
                    N=2, C_in=groups * cig, C_out=groups * cog, groups=groups, L=L, k=k,
                    stride=s, padding_before=pb, padding_after=pa, dilation=d, output_padding=op,
                    has_bias=bool(rng.integers(0, 2))))
    return cases


CASES = _cases()


@pytest.mark.parametrize("wl", CASES, ids=lambda wl: f"{wl.name}-r{len(wl.x_shape)-2}"
                         f"{'T' if wl.transposed else 'F'}")
def test_values_match_torch_float64(oracle_mod, wl):
    x, w, b = synth.make_inputs(wl)
    kw = kw_of(wl)
    y, A = oracle_mod.conv(as64(x), as64(w), as64(b), **kw)
    ref = torch_ref(as64(x), as64(w), as64(b), **kw)
    assert y.shape == ref.shape
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)
    # A is the same convolution applied to |x| and |w|, plus |b|.
    refA = torch_ref(np.abs(as64(x)), np.abs(as64(w)), None if b is None else np.abs(as64(b)),
                     **kw)
    np.testing.assert_allclose(A, refA, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("wl", CASES[::3], ids=lambda wl: wl.name)
def test_out_shape_matches_torch(oracle_mod, wl):
    x, w, b = synth.make_inputs(wl)
    kw = kw_of(wl)
    ref = torch_ref(as64(x), as64(w), None, **kw)
    assert oracle_mod.out_shape(tuple(x.shape), tuple(w.shape), **kw) == ref.shape


def test_symmetric_padding_shapes_match_torch_directly(oracle_mod):
    """Shapes straight from torch's own padding/output_padding arguments."""
    for r in (1, 2, 3):
        x = torch.zeros((1, 2) + (7,) * r, dtype=torch.float64)
        for k, s, p, d in [(3, 1, 1, 1), (3, 2, 1, 1), (5, 3, 2, 2), (2, 2, 0, 1), (4, 2, 1, 1)]:
            w = torch.zeros((4, 2) + (k,) * r, dtype=torch.float64)
            y = CONV[r](x, w, stride=s, padding=p, dilation=d)
            assert oracle_mod.out_shape(tuple(x.shape), tuple(w.shape), stride=s,
                                        padding_before=p, padding_after=p, dilation=d) == \
                tuple(y.shape)
            for op in range(max(s, d)):
                wt = torch.zeros((2, 4) + (k,) * r, dtype=torch.float64)
                yt = CONVT[r](x, wt, stride=s, padding=p, output_padding=op, dilation=d)
                assert oracle_mod.out_shape(tuple(x.shape), tuple(wt.shape), stride=s,
                                            padding_before=p, padding_after=p, dilation=d,
                                            transposed=True, output_padding=op) == tuple(yt.shape)


def test_out_len_rejects_empty_output(oracle_mod):
    assert oracle_mod.out_len(False, 2, 5, 1, 0, 0, 1, 0) == -1
    assert oracle_mod.out_len(False, 2, 5, 1, 1, 2, 1, 0) == 1
    assert oracle_mod.out_len(True, 1, 1, 1, 1, 0, 1, 0) == -1


# --------------------------------------------------------- closed forms --

@pytest.mark.parametrize("transposed", [False, True])
@pytest.mark.parametrize("geom", [
    dict(L=(9,), k=(4,), s=(2,), pb=(1,), pa=(2,), d=(1,)),
    dict(L=(6, 7), k=(3, 2), s=(1, 3), pb=(2, 0), pa=(0, 1), d=(2, 1)),
    dict(L=(4, 3, 5), k=(2, 3, 2), s=(2, 1, 2), pb=(1, 1, 0), pa=(0, 1, 1), d=(1, 1, 2)),
])
def test_delta_kernel_closed_form(oracle_mod, transposed, geom):
    """A one-hot kernel at tap t0 copies (shifted) input values: forward
    y[o] = x[o*s - pb + t0*d]; transposed y[o] = x[(o + pb - t0*d)/s] when
    that is an exact in-range quotient; 0 elsewhere, plus the bias."""
    r = len(geom["L"])
    C = 3
    rng = np.random.default_rng(3)
    x = rng.standard_normal((2, C) + geom["L"])
    b = rng.standard_normal(C)
    op = tuple(0 for _ in range(r))
    if transposed:
        op = tuple(min(1, max(si, di) - 1) for si, di in zip(geom["s"], geom["d"]))
    for t0 in np.ndindex(*geom["k"]):
        w = np.zeros((C, 1) + geom["k"])
        w[(slice(None), 0) + t0] = 1.0
        y, _ = oracle_mod.conv(x, w, b, stride=geom["s"], padding_before=geom["pb"],
                               padding_after=geom["pa"], dilation=geom["d"], groups=C,
                               transposed=transposed, output_padding=op)
        expect = np.empty_like(y)
        for idx in np.ndindex(*y.shape):
            n, c, o = idx[0], idx[1], idx[2:]
            src = []
            for dd in range(r):
                if not transposed:
                    i = o[dd] * geom["s"][dd] - geom["pb"][dd] + t0[dd] * geom["d"][dd]
                    ok = 0 <= i < geom["L"][dd]
                else:
                    num = o[dd] + geom["pb"][dd] - t0[dd] * geom["d"][dd]
                    i = num // geom["s"][dd]
                    ok = num >= 0 and num % geom["s"][dd] == 0 and i < geom["L"][dd]
                if not ok:
                    src = None
                    break
                src.append(i)
            expect[idx] = b[c] + (x[(n, c) + tuple(src)] if src is not None else 0.0)
        np.testing.assert_array_equal(y, expect)


def _count_valid(transposed, o, L, k, s, pb, d):
    """Number of taps t in [0, k) that reach an input position, by interval
    arithmetic (forward) or by stepping through the residue class (transposed)."""
    if not transposed:
        # 0 <= o*s - pb + t*d <= L-1  <=>  t in [ceil((pb - o*s)/d), floor((L-1+pb-o*s)/d)]
        lo = -((o * s - pb) // d)
        hi = (L - 1 + pb - o * s) // d
        return max(0, min(hi, k - 1) - max(lo, 0) + 1)
    count = 0
    for i in range(L):                       # input i reaches o via t = (o + pb - i*s)/d
        num = o + pb - i * s
        if num >= 0 and num % d == 0 and num // d < k:
            count += 1
    return count


@pytest.mark.parametrize("transposed", [False, True])
def test_all_ones_counts(oracle_mod, transposed):
    L, k, s, pb, pa, d = (7, 5), (3, 4), (2, 1), (1, 3), (2, 0), (1, 2)
    groups, cig, cog = 2, 3, 2
    x = np.ones((1, groups * cig) + L)
    wshape = ((groups * cig, cog) if transposed else (groups * cog, cig)) + k
    w = np.ones(wshape)
    op = (1, 1) if transposed else (0, 0)
    y, A = oracle_mod.conv(x, w, None, stride=s, padding_before=pb, padding_after=pa,
                           dilation=d, groups=groups, transposed=transposed, output_padding=op)
    for idx in np.ndindex(*y.shape):
        o = idx[2:]
        cnt = cig
        for dd in range(2):
            cnt *= _count_valid(transposed, o[dd], L[dd], k[dd], s[dd], pb[dd], d[dd])
        assert y[idx] == cnt and A[idx] == cnt


# ----------------------------------------------------------- identities --

@pytest.mark.parametrize("seed", range(6))
def test_adjoint_identity(oracle_mod, seed):
    """<conv(x, w), z> == <x, convT(z, w)> with the same weight tensor."""
    rng = np.random.default_rng(seed)
    r = 1 + seed % 3
    groups = 1 + seed % 2
    cig, cog = 2, 3
    L = tuple(int(v) for v in rng.integers(4, 8, r))
    k = tuple(int(v) for v in rng.integers(1, 4, r))
    s = tuple(int(v) for v in rng.integers(1, 4, r))
    d = tuple(int(v) for v in rng.integers(1, 3, r))
    pb = tuple(int(v) for v in rng.integers(0, 3, r))
    pa = tuple(int(v) for v in rng.integers(0, 3, r))
    x = rng.standard_normal((2, groups * cig) + L)
    w = rng.standard_normal((groups * cog, cig) + k)
    y, _ = oracle_mod.conv(x, w, None, stride=s, padding_before=pb, padding_after=pa,
                           dilation=d, groups=groups)
    op = tuple((L[i] + pb[i] + pa[i] - d[i] * (k[i] - 1) - 1) % s[i] for i in range(r))
    z = rng.standard_normal(y.shape)
    xt, _ = oracle_mod.conv(z, w, None, stride=s, padding_before=pb, padding_after=pa,
                            dilation=d, groups=groups, transposed=True, output_padding=op)
    assert xt.shape == x.shape
    lhs = float(np.sum(y * z))
    rhs = float(np.sum(x * xt))
    assert abs(lhs - rhs) <= 1e-12 * max(1.0, float(np.sum(np.abs(y * z))))


@pytest.mark.parametrize("geom", [
    dict(L=(5,), k=(3,), s=(2,), pb=(1,), pa=(1,), d=(1,), groups=1),
    dict(L=(4, 3), k=(2, 2), s=(1, 2), pb=(0, 1), pa=(1, 0), d=(2, 1), groups=2),
    dict(L=(3, 2, 3), k=(2, 1, 2), s=(2, 1, 1), pb=(1, 0, 0), pa=(0, 0, 1), d=(1, 1, 1), groups=1),
])
def test_operator_matrix_transpose(oracle_mod, geom):
    """Exhaustive: build the forward operator from unit impulses; the
    transposed operator (same w) must be exactly its transpose."""
    r = len(geom["L"])
    G = geom["groups"]
    cig, cog = 2, 2
    rng = np.random.default_rng(11)
    w = rng.integers(-9, 10, (G * cog, cig) + geom["k"]).astype(float)
    kw = dict(stride=geom["s"], padding_before=geom["pb"], padding_after=geom["pa"],
              dilation=geom["d"], groups=G)
    xshape = (1, G * cig) + geom["L"]
    y0, _ = oracle_mod.conv(np.zeros(xshape), w, None, **kw)
    nin, nout = int(np.prod(xshape)), y0.size
    M = np.zeros((nout, nin))
    for j in range(nin):
        e = np.zeros(nin)
        e[j] = 1.0
        M[:, j] = oracle_mod.conv(e.reshape(xshape), w, None, **kw)[0].ravel()
    op = tuple((geom["L"][i] + geom["pb"][i] + geom["pa"][i] - geom["d"][i] * (geom["k"][i] - 1)
                - 1) % geom["s"][i] for i in range(r))
    MT = np.zeros((nin, nout))
    for j in range(nout):
        e = np.zeros(nout)
        e[j] = 1.0
        MT[:, j] = oracle_mod.conv(e.reshape(y0.shape), w, None, transposed=True,
                                   output_padding=op, **kw)[0].ravel()
    np.testing.assert_array_equal(MT, M.T)
    assert np.count_nonzero(M) > 0


@pytest.mark.parametrize("s", [1, 2, 3])
def test_transposed_equals_zero_inserted_flipped_forward(oracle_mod, s):
    """Textbook rewrite (the backend's rewrite of transposed convolutions as
    convolutions): insert s-1 zeros between inputs, swap the weight's first two
    axes within each group, flip the taps, and pad by d*(k-1) - pb before and
    d*(k-1) - pa + op after."""
    rng = np.random.default_rng(s)
    G, cig, cog = 2, 2, 3
    L, k, d, pb, pa = (6, 5), (3, 2), (1, 2), (1, 2), (2, 0)
    op = tuple(min(1, max(s, di) - 1) for di in d)
    x = rng.standard_normal((2, G * cig) + L)
    w = rng.standard_normal((G * cig, cog) + k)
    b = rng.standard_normal(G * cog)
    y, _ = oracle_mod.conv(x, w, b, stride=s, padding_before=pb, padding_after=pa, dilation=d,
                           groups=G, transposed=True, output_padding=op)
    up = np.zeros((2, G * cig) + tuple((Li - 1) * s + 1 for Li in L))
    up[:, :, ::s, ::s] = x
    wf = np.zeros((G * cog, cig) + k)
    for g in range(G):
        for j in range(cog):
            for c in range(cig):
                wf[g * cog + j, c] = w[g * cig + c, j][::-1, ::-1]
    pbf = tuple(d[i] * (k[i] - 1) - pb[i] for i in range(2))
    paf = tuple(d[i] * (k[i] - 1) - pa[i] + op[i] for i in range(2))
    assert min(pbf + paf) >= 0
    yf, _ = oracle_mod.conv(up, wf, b, stride=1, padding_before=pbf, padding_after=paf,
                            dilation=d, groups=G)
    np.testing.assert_allclose(y, yf, rtol=1e-13, atol=1e-13)


def test_one_by_one_is_matmul(oracle_mod):
    rng = np.random.default_rng(5)
    x = rng.standard_normal((3, 6, 4, 5))
    w = rng.standard_normal((7, 6, 1, 1))
    b = rng.standard_normal(7)
    y, _ = oracle_mod.conv(x, w, b)
    xm = x.transpose(0, 2, 3, 1).reshape(-1, 6)
    ref = (xm @ w[:, :, 0, 0].T + b).reshape(3, 4, 5, 7).transpose(0, 3, 1, 2)
    np.testing.assert_allclose(y, ref, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("transposed", [False, True])
def test_groups_are_independent_dense_convs(oracle_mod, transposed):
    rng = np.random.default_rng(9)
    G, cig, cog = 3, 2, 4
    x = rng.standard_normal((2, G * cig, 6, 5))
    w = rng.standard_normal(((G * cig, cog) if transposed else (G * cog, cig)) + (3, 2))
    b = rng.standard_normal(G * cog)
    kw = dict(stride=(2, 1), padding_before=(1, 0), padding_after=(0, 1), dilation=(1, 2),
              transposed=transposed, output_padding=(1, 0) if transposed else (0, 0))
    y, _ = oracle_mod.conv(x, w, b, groups=G, **kw)
    parts = []
    for g in range(G):
        xs = x[:, g * cig:(g + 1) * cig]
        ws = w[g * cig:(g + 1) * cig] if transposed else w[g * cog:(g + 1) * cog]
        parts.append(oracle_mod.conv(xs, ws, b[g * cog:(g + 1) * cog], groups=1, **kw)[0])
    np.testing.assert_array_equal(y, np.concatenate(parts, axis=1))


def test_bias_is_separable(oracle_mod):
    rng = np.random.default_rng(2)
    x = rng.standard_normal((2, 4, 7))
    w = rng.standard_normal((6, 2, 3))
    b = rng.standard_normal(6)
    y1, A1 = oracle_mod.conv(x, w, b, groups=2, padding_before=1, padding_after=2)
    y0, A0 = oracle_mod.conv(x, w, None, groups=2, padding_before=1, padding_after=2)
    np.testing.assert_allclose(y1 - y0, np.broadcast_to(b[None, :, None], y0.shape), atol=1e-12)
    np.testing.assert_allclose(A1 - A0, np.broadcast_to(np.abs(b)[None, :, None], y0.shape),
                               atol=1e-12)


def test_points_match_full_output(oracle_mod):
    rng = np.random.default_rng(4)
    x = rng.standard_normal((2, 6, 9, 8))
    w = rng.standard_normal((6, 4, 3, 2))
    b = rng.standard_normal(12)
    kw = dict(stride=(2, 1), padding_before=(1, 0), padding_after=(1, 1), dilation=(1, 2),
              groups=3, transposed=True, output_padding=(1, 0))
    y, A = oracle_mod.conv(x, w, b, **kw)
    pts = np.stack([rng.integers(0, n, 50) for n in y.shape], axis=1)
    yp, Ap = oracle_mod.conv_points(x, w, b, pts, **kw)
    np.testing.assert_array_equal(yp, y[tuple(pts.T)])
    np.testing.assert_array_equal(Ap, A[tuple(pts.T)])


# --------------------------------------------------------------- layout --

@pytest.mark.parametrize("r", [1, 2, 3])
@pytest.mark.parametrize("xl", ["contiguous", "channels_last"])
@pytest.mark.parametrize("wl", ["contiguous", "channels_last"])
@pytest.mark.parametrize("transposed", [False, True])
def test_out_strides_match_torch_cpu(oracle_mod, r, xl, wl, transposed):
    """CPU ATen's convolution (fp32: its channels-last-aware path) returns
    the layout of the rule for every rank and both layouts of x and w: 1-D
    calls ignore an NLC x (ATen makes x contiguous before running the call as
    2-D) but follow an NLC weight."""
    x = torch.randn((2, 4) + (5,) * r, dtype=torch.float32)
    if xl == "channels_last":
        x = synth.channels_last_copy(x)
    w = torch.randn(((4, 3) if transposed else (6, 4)) + (3,) * r, dtype=torch.float32)
    if wl == "channels_last":
        w = synth.channels_last_copy(w)
    y = (CONVT if transposed else CONV)[r](x, w, stride=2, padding=1)
    assert oracle_mod.out_strides(tuple(y.shape), tuple(x.shape), tuple(x.stride()),
                                  tuple(w.shape), tuple(w.stride())) == tuple(y.stride())


def test_out_strides_rule_cases(oracle_mod):
    # 1-D: an NLC input with a contiguous weight -> contiguous output (the
    # transposed 1-D upsampling workload's layout)
    assert oracle_mod.out_strides((16, 512, 16383), (16, 512, 8192), (4194304, 1, 512),
                                  (512, 512, 4), (2048, 4, 1)) == (8388096, 16383, 1)
    # 1-D: an NLC weight -> NLC output
    assert oracle_mod.out_strides((2, 6, 20), (2, 8, 20), (160, 20, 1),
                                  (6, 8, 3), (24, 1, 8)) == (120, 1, 6)
    # C == 1: both formats describe x -> contiguous
    assert oracle_mod.out_strides((2, 3, 4, 4), (2, 1, 4, 4), (16, 16, 4, 1),
                                  (3, 1, 1, 1), (1, 1, 1, 1)) == (48, 16, 4, 1)
    # channels-last weight makes the output channels-last
    assert oracle_mod.out_strides((2, 8, 4, 4), (2, 3, 4, 4), (48, 16, 4, 1),
                                  (8, 3, 3, 3), (27, 1, 9, 3)) == (128, 1, 32, 8)
    # NDHWC input -> NDHWC output
    assert oracle_mod.out_strides((2, 6, 3, 3, 3), (2, 4, 5, 5, 5), (500, 1, 100, 20, 4),
                                  (6, 4, 3, 3, 3), (108, 27, 9, 3, 1)) == (162, 1, 54, 18, 6)
    # a channel slice of a channels-last tensor is still channels-last-like
    assert oracle_mod.out_strides((2, 3, 4, 4), (2, 4, 4, 4), (128, 1, 32, 8),
                                  (3, 4, 1, 1), (4, 1, 1, 1)) == (48, 1, 12, 3)
    # zero-size batch: contiguous, products over max(size, 1)
    assert oracle_mod.out_strides((0, 5, 3), (0, 5, 3), (15, 3, 1), (5, 5, 1),
                                  (5, 1, 1)) == (15, 3, 1)


# ------------------------------------------------------------- gradients --

def _torch_fn(x, w, b, *, stride, padding_before, padding_after, dilation, groups, transposed, output_padding):
    """The op as differentiable torch CPU float64 ops (asymmetric padding by an
    explicit pad for forward calls, a crop of the uncropped output for
    transposed ones)."""
    r = x.dim() - 2
    if not transposed:
        pads = []
        for i in reversed(range(r)):
            pads += [padding_before[i], padding_after[i]]
        y = CONV[r](F.pad(x, pads), w, None, stride=tuple(stride), padding=0, dilation=tuple(dilation),
                    groups=groups)
    else:
        full = CONVT[r](x, w, None, stride=tuple(stride), padding=0, output_padding=0, groups=groups,
                        dilation=tuple(dilation))
        ext = []
        for i in reversed(range(r)):
            ext += [0, output_padding[i]]
        full = F.pad(full, ext)
        sl = [slice(None), slice(None)]
        for i in range(r):
            L_full = full.shape[2 + i] - output_padding[i]
            sl.append(slice(padding_before[i], L_full - padding_after[i] + output_padding[i]))
        y = full[tuple(sl)]
    if b is not None:
        y = y + b.reshape((1, -1) + (1,) * r)
    return y


@pytest.mark.parametrize("wl", CASES, ids=lambda wl: f"{wl.name}-r{len(wl.x_shape)-2}"
                         f"{'T' if wl.transposed else 'F'}")
def test_gradients_match_torch_autograd(oracle_mod, wl):
    """dx, dw, db against torch CPU float64 autograd of the same op, for
    forward and transposed calls of every rank (groups, dilation, strides,
    asymmetric padding, output_padding)."""
    x, w, b = synth.make_inputs(wl)
    kw = kw_of(wl)
    xt = x.double().requires_grad_(True)
    wt = w.double().requires_grad_(True)
    bt = b.double().requires_grad_(True) if b is not None else None
    y = _torch_fn(xt, wt, bt, **kw)
    gy = torch.randn(y.shape, dtype=torch.float64, generator=torch.Generator().manual_seed(wl.seed))
    y.backward(gy)
    dx, Adx, dw, Adw, db, Adb = oracle_mod.conv_backward(as64(x), as64(w), gy.numpy(), with_bias=b is not None,
                                                         **kw)
    np.testing.assert_allclose(dx, xt.grad.numpy(), rtol=0, atol=1e-12 * (1 + Adx.max()))
    np.testing.assert_allclose(dw, wt.grad.numpy(), rtol=0, atol=1e-12 * (1 + Adw.max()))
    if b is not None:
        np.testing.assert_allclose(db, bt.grad.numpy(), rtol=0, atol=1e-12 * (1 + Adb.max()))
    # The bounds are the same sums over absolute values.
    assert np.all(Adx >= np.abs(dx) - 1e-12) and np.all(Adw >= np.abs(dw) - 1e-12)


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("transposed", [False, True])
def test_gradient_adjoint_identities(oracle_mod, seed, transposed):
    """For the bias-free op f(x, w), linear in each argument,
    <f(x, w), gy> = <x, dx> = <w, dw>, and <1, gy> = sum(db)."""
    rng = np.random.default_rng(40 + seed)
    r = 1 + seed % 3
    groups = 1 + seed % 2
    cig, cog = 2, 3
    L = tuple(int(v) for v in rng.integers(4, 8, r))
    k = tuple(int(v) for v in rng.integers(1, 4, r))
    s = tuple(int(v) for v in rng.integers(1, 4, r))
    d = tuple(int(v) for v in rng.integers(1, 3, r))
    pb = tuple(int(v) for v in rng.integers(0, 3, r))
    pa = tuple(int(v) for v in rng.integers(0, 3, r))
    op = tuple(int(rng.integers(0, max(si, di))) for si, di in zip(s, d)) if transposed else (0,) * r
    x = rng.standard_normal((2, groups * cig) + L)
    w = rng.standard_normal(((groups * cig, cog) if transposed else (groups * cog, cig)) + k)
    kw = dict(stride=s, padding_before=pb, padding_after=pa, dilation=d, groups=groups, transposed=transposed,
              output_padding=op)
    try:
        y, _ = oracle_mod.conv(x, w, None, **kw)
    except ValueError:
        pytest.skip("empty output for this draw")
    gy = rng.standard_normal(y.shape)
    dx, _, dw, _, db, _ = oracle_mod.conv_backward(x, w, gy, **kw)
    f = float(np.sum(y * gy))
    scale = max(1.0, float(np.sum(np.abs(y * gy))))
    assert abs(float(np.sum(x * dx)) - f) <= 1e-12 * scale
    assert abs(float(np.sum(w * dw)) - f) <= 1e-12 * scale
    assert abs(float(np.sum(db)) - float(np.sum(gy))) <= 1e-12 * max(1.0, float(np.sum(np.abs(gy))))


@pytest.mark.parametrize("transposed", [False, True])
def test_gradients_brute_force(oracle_mod, transposed):
    """Tiny shapes, integer values: dx = M^T gy and dw = Mw^T gy exactly,
    with M and Mw the op's matrices in x and in w built column by column
    from unit impulses through the (separately pinned) forward op."""
    rng = np.random.default_rng(5)
    kw = dict(stride=(2, 1), padding_before=(1, 0), padding_after=(0, 1), dilation=(1, 2), groups=2,
              transposed=transposed, output_padding=(1, 0) if transposed else (0, 0))
    x = rng.integers(-5, 6, (2, 4, 3, 4)).astype(float)
    w = rng.integers(-5, 6, (4, 3, 2, 2) if transposed else (6, 2, 2, 2)).astype(float)
    y, _ = oracle_mod.conv(x, w, None, **kw)
    gy = rng.integers(-5, 6, y.shape).astype(float)
    dx, _, dw, _, db, _ = oracle_mod.conv_backward(x, w, gy, **kw)
    for arr, grad, which in ((x, dx, "x"), (w, dw, "w")):
        exp = np.zeros(arr.size)
        for j in range(arr.size):
            e = np.zeros(arr.size)
            e[j] = 1.0
            col = oracle_mod.conv(e.reshape(arr.shape) if which == "x" else x,
                                  w if which == "x" else e.reshape(arr.shape), None, **kw)[0]
            exp[j] = float(np.sum(col * gy))
        np.testing.assert_array_equal(grad.ravel(), exp, err_msg=which)
    np.testing.assert_array_equal(db, gy.sum(axis=(0, 2, 3)))
