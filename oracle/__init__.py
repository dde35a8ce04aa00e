"""Double-precision reference convolution -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never loads it, and
this package imports nothing from the product: the two share no code.

Contents
  * ``out_len`` / ``out_shape``: output sizes of the canonical op.
  * ``out_strides``: the output memory format (dense, channels-last or
    contiguous) -- see ``out_strides`` for the reading.
  * ``conv``: full output and per-element bound A, computed by ``oracle.c``.
  * ``conv_points``: the same for selected output elements only.
  * ``conv_backward``: the input, weight and bias gradients for a given
    output gradient, each with its bound.

Semantics follow executorch PR #25084 ("Add triton::convolution and the conv
routing framework", description), the forward index map printed in
torch/_inductor/kernel/conv.py (LOOP_BODY_2D), and the transposed gather of
executorch PR #25091 ("Run transposed convolutions on the implicit-GEMM
template", description, second paragraph).  ``oracle.c`` states each.

Parity status: every function here is pinned by ``tests/test_oracle_pins.py``
(library routines, closed forms, identities, hand-derived fixtures).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    """Compile ``oracle.c`` into ``liboracle.so`` (gcc, OpenMP, -O2)."""
    cmd = ["gcc", "-std=c99", "-O2", "-fopenmp", "-fPIC", "-shared", _SRC,
           "-o", _LIB_PATH + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.check_call(cmd)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


class _Geom(ctypes.Structure):
    _fields_ = [
        ("rank", ctypes.c_int32), ("transposed", ctypes.c_int32),
        ("N", ctypes.c_int64), ("C_in", ctypes.c_int64),
        ("C_out", ctypes.c_int64), ("groups", ctypes.c_int64),
        ("L", ctypes.c_int64 * 3), ("K", ctypes.c_int64 * 3),
        ("O", ctypes.c_int64 * 3), ("s", ctypes.c_int64 * 3),
        ("pb", ctypes.c_int64 * 3), ("pa", ctypes.c_int64 * 3),
        ("d", ctypes.c_int64 * 3), ("op", ctypes.c_int64 * 3),
    ]


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        dp = ctypes.POINTER(ctypes.c_double)
        lib.oracle_conv_f64.argtypes = [ctypes.POINTER(_Geom), dp, dp, dp, dp, dp, ctypes.c_int]
        lib.oracle_conv_f64.restype = ctypes.c_int
        lib.oracle_conv_points_f64.argtypes = [ctypes.POINTER(_Geom), dp, dp, dp, ctypes.c_int64,
                                               ctypes.POINTER(ctypes.c_int64), dp, dp, ctypes.c_int]
        lib.oracle_conv_points_f64.restype = ctypes.c_int
        lib.oracle_out_len.argtypes = [ctypes.c_int32] + [ctypes.c_int64] * 7
        lib.oracle_out_len.restype = ctypes.c_int64
        lib.oracle_conv_backward_f64.argtypes = [ctypes.POINTER(_Geom), dp, dp, dp, dp, dp, dp, dp, dp, dp,
                                                 ctypes.c_int]
        lib.oracle_conv_backward_f64.restype = ctypes.c_int
        lib.oracle_max_threads.argtypes = []
        lib.oracle_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def max_threads() -> int:
    """Threads the oracle's OpenMP regions use."""
    return int(_load().oracle_max_threads())


def _per_dim(v, r: int, default: int) -> Tuple[int, ...]:
    if v is None:
        return (default,) * r
    if isinstance(v, (int, np.integer)):
        return (int(v),) * r
    v = tuple(int(a) for a in v)
    if len(v) == 1:
        return v * r
    if len(v) != r:
        raise ValueError(f"expected {r} values, got {v}")
    return v


def out_len(transposed: bool, L: int, k: int, s: int, pb: int, pa: int, d: int, op: int) -> int:
    """Output length of one spatial dimension (-1 when it would be < 1).

    forward:     floor((L + pb + pa - d*(k-1) - 1) / s) + 1
    transposed:  (L-1)*s - pb - pa + d*(k-1) + op + 1
    (The pages name ATen's layout as the target but print no formula; these
    are ATen's formulas with 2*padding split into pb + pa.)
    """
    return int(_load().oracle_out_len(int(bool(transposed)), L, k, s, pb, pa, d, op))


def out_shape(x_shape: Sequence[int], w_shape: Sequence[int], *, stride=1, padding_before=0,
              padding_after=0, dilation=1, groups=1, transposed=False, output_padding=0):
    """Batched output shape [N, C_out, O...] for batched x and w shapes."""
    r = len(x_shape) - 2
    s = _per_dim(stride, r, 1)
    pb = _per_dim(padding_before, r, 0)
    pa = _per_dim(padding_after, r, 0)
    d = _per_dim(dilation, r, 1)
    op = _per_dim(output_padding, r, 0)
    c_out = w_shape[1] * groups if transposed else w_shape[0]
    outs = [out_len(transposed, x_shape[2 + i], w_shape[2 + i], s[i], pb[i], pa[i], d[i], op[i])
            for i in range(r)]
    return (x_shape[0], c_out, *outs)


def _ordered_like(sizes: Sequence[int], strides: Sequence[int], order: Sequence[int]) -> bool:
    """True when the dims listed in ``order`` (fastest first) nest without
    overlap: each dim of size > 1 has a stride at least the extent of the
    faster dims before it.  Size-1 dims are ignored; any size 0 -> False."""
    if any(int(s) == 0 for s in sizes):
        return False
    end = 0
    for dim in order:
        if sizes[dim] == 1:
            continue
        if strides[dim] < end or strides[dim] <= 0:
            return False
        end = strides[dim] * sizes[dim]
    return True


def is_channels_last(sizes: Sequence[int], strides: Sequence[int]) -> bool:
    """Channels-last-like and not also contiguous-like (rank = 2 + spatial)."""
    nd = len(sizes)
    cl = [1] + list(range(nd - 1, 1, -1)) + [0]          # C, L_r .. L_1, N
    contig = list(range(nd - 1, 1, -1)) + [1, 0]          # L_r .. L_1, C, N
    return _ordered_like(sizes, strides, cl) and not _ordered_like(sizes, strides, contig)


def out_strides(y_shape: Sequence[int], x_sizes: Sequence[int], x_strides: Sequence[int],
                w_sizes: Sequence[int], w_strides: Sequence[int]) -> Tuple[int, ...]:
    """Element strides of the output (batched shapes).

    Reading of the output layout the pages name (executorch PR #25084, "Add
    triton::convolution and the conv routing framework", description: the op
    returns the layout ATen's convolution returns).  The output is dense.  For
    2-D and 3-D calls it is channels-last (C fastest, then the last spatial
    dim, ..., then N) when x or w is channels-last-like and not also
    contiguous-like, and contiguous otherwise.  ATen runs a 1-D call as a 2-D
    one with H = 1 after making x contiguous, so for 1-D calls only w counts:
    an NLC x alone gives a contiguous output.  Products use max(size, 1), as
    ATen does for empty dims.
    """
    nd = len(y_shape)
    x_counts = nd >= 4
    if (x_counts and is_channels_last(x_sizes, x_strides)) or is_channels_last(w_sizes, w_strides):
        order = [1] + list(range(nd - 1, 1, -1)) + [0]
    else:
        order = list(range(nd - 1, -1, -1))
    st = [0] * nd
    acc = 1
    for dim in order:
        st[dim] = acc
        acc *= max(int(y_shape[dim]), 1)
    return tuple(st)


def _geom(x: np.ndarray, w: np.ndarray, stride, padding_before, padding_after, dilation, groups,
          transposed, output_padding) -> _Geom:
    r = x.ndim - 2
    if r < 1 or r > 3 or w.ndim != x.ndim:
        raise ValueError("x and w must be [N, C, L...] / [.., .., k...] with 1..3 spatial dims")
    s = _per_dim(stride, r, 1)
    pb = _per_dim(padding_before, r, 0)
    pa = _per_dim(padding_after, r, 0)
    d = _per_dim(dilation, r, 1)
    op = _per_dim(output_padding, r, 0)
    g = _Geom()
    g.rank = r
    g.transposed = int(bool(transposed))
    g.N, g.C_in = x.shape[0], x.shape[1]
    g.groups = groups
    g.C_out = w.shape[1] * groups if transposed else w.shape[0]
    for i in range(3):
        if i < r:
            g.L[i], g.K[i] = x.shape[2 + i], w.shape[2 + i]
            g.s[i], g.pb[i], g.pa[i], g.d[i], g.op[i] = s[i], pb[i], pa[i], d[i], op[i]
            g.O[i] = out_len(transposed, g.L[i], g.K[i], s[i], pb[i], pa[i], d[i], op[i])
            if g.O[i] < 1:
                raise ValueError("output length < 1")
        else:
            g.L[i] = g.K[i] = g.O[i] = g.s[i] = g.d[i] = 1
            g.pb[i] = g.pa[i] = g.op[i] = 0
    if x.shape[1] % groups or g.C_out % groups:
        raise ValueError("channels not divisible by groups")
    wi = x.shape[1] if transposed else g.C_out
    if w.shape[0] != wi or (not transposed and w.shape[1] != x.shape[1] // groups):
        raise ValueError("weight shape does not match")
    return g


def _dptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _prep(a: Optional[np.ndarray]) -> Optional[np.ndarray]:
    if a is None:
        return None
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def conv(x, w, b=None, *, stride=1, padding_before=0, padding_after=0, dilation=1, groups=1,
         transposed=False, output_padding=0, nthreads: int = 0):
    """Full canonical convolution in float64.

    x: [N, C_in, L...]; w: [C_out, C_in/groups, k...] (forward) or
    [C_in, C_out/groups, k...] (transposed); b: [C_out] or None.
    Returns (y, A), both [N, C_out, O...] float64, A = sum|x*w| + |b|.
    """
    x, w, b = _prep(x), _prep(w), _prep(b)
    g = _geom(x, w, stride, padding_before, padding_after, dilation, groups, transposed,
              output_padding)
    shape = (g.N, g.C_out) + tuple(g.O[i] for i in range(g.rank))
    y = np.empty(shape, dtype=np.float64)
    A = np.empty(shape, dtype=np.float64)
    if y.size:
        rc = _load().oracle_conv_f64(ctypes.byref(g), _dptr(x), _dptr(w),
                                     _dptr(b) if b is not None else None, _dptr(y), _dptr(A),
                                     int(nthreads))
        if rc != 0:
            raise ValueError("oracle rejected the geometry")
    return y, A


def conv_points(x, w, b, points, *, stride=1, padding_before=0, padding_after=0, dilation=1,
                groups=1, transposed=False, output_padding=0, nthreads: int = 0):
    """Selected outputs.  ``points`` is an int array [P, 2 + r] of
    (n, c_out, o...) indices.  Returns (y, A) of shape [P]."""
    x, w, b = _prep(x), _prep(w), _prep(b)
    g = _geom(x, w, stride, padding_before, padding_after, dilation, groups, transposed,
              output_padding)
    pts = np.asarray(points, dtype=np.int64)
    P = pts.shape[0]
    idx = np.zeros((P, 5), dtype=np.int64)
    idx[:, : pts.shape[1]] = pts
    idx = np.ascontiguousarray(idx)
    y = np.empty(P, dtype=np.float64)
    A = np.empty(P, dtype=np.float64)
    if P:
        rc = _load().oracle_conv_points_f64(
            ctypes.byref(g), _dptr(x), _dptr(w), _dptr(b) if b is not None else None,
            ctypes.c_int64(P), idx.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
            _dptr(y), _dptr(A), int(nthreads))
        if rc != 0:
            raise ValueError("oracle rejected the geometry or a point")
    return y, A


def conv_backward(x, w, gy, *, with_bias=True, stride=1, padding_before=0, padding_after=0, dilation=1,
                  groups=1, transposed=False, output_padding=0, nthreads: int = 0):
    """Gradients of the canonical op for an output gradient ``gy`` (float64).

    Returns (dx, Adx, dw, Adw, db, Adb): dx like x, dw like w, db [C_out]
    (None when ``with_bias`` is false), each with the sum of the absolute
    values of its terms.  Follows the backward of the convolution lowering in
    torch/_inductor/kernel/conv.py (convolution_backward): input, weight and
    bias gradients of the same op, stated in ``oracle.c``.
    """
    x, w, gy = _prep(x), _prep(w), _prep(gy)
    g = _geom(x, w, stride, padding_before, padding_after, dilation, groups, transposed, output_padding)
    shape = (g.N, g.C_out) + tuple(g.O[i] for i in range(g.rank))
    if gy.shape != shape:
        raise ValueError(f"gy has shape {gy.shape}, the output is {shape}")
    dx, Adx = np.empty_like(x), np.empty_like(x)
    dw, Adw = np.empty_like(w), np.empty_like(w)
    db = np.empty(g.C_out) if with_bias else None
    Adb = np.empty(g.C_out) if with_bias else None
    rc = _load().oracle_conv_backward_f64(ctypes.byref(g), _dptr(x), _dptr(w), _dptr(gy), _dptr(dx), _dptr(Adx),
                                          _dptr(dw), _dptr(Adw), _dptr(db) if with_bias else None,
                                          _dptr(Adb) if with_bias else None, int(nthreads))
    if rc != 0:
        raise ValueError("oracle rejected the geometry")
    return dx, Adx, dw, Adw, db, Adb
