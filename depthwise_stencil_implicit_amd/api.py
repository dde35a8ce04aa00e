"""Python binding of the canonical convolution (argument marshalling only).

``conv_bind``, ``conv_out_shape``, ``conv_plan`` and ``conv_run`` wrap the C
ABI calls of the same names one to one.  ``conv`` chains them for torch
tensors on the GPU: torch provides the device memory (output, workspace) and
the current HIP stream; every step of the computation runs in the library's
kernels.  The ATen-style helpers (``conv1d`` ... ``_convolution``) only
translate ATen's arguments into the canonical ones (executorch PR #25084,
"Add triton::convolution and the conv routing framework", description: every
ATen convolution overload maps onto the one canonical op).
"""
from __future__ import annotations

import ctypes
from typing import Optional, Sequence, Tuple, Union

import torch

from . import _abi as A

_TORCH_DT = {torch.float32: A.F32, torch.float16: A.F16, torch.bfloat16: A.BF16}


class ConvError(RuntimeError):
    def __init__(self, status: int, msg: str = ""):
        self.status = status
        name = A.lib().conv_status_string(status).decode()
        super().__init__(f"{name}" + (f": {msg}" if msg else ""))


def _check(status: int, msg: str = "") -> None:
    if status != A.OK:
        raise ConvError(status, msg)


# ---------------------------------------------------------------- descriptors --

def describe(t: Optional[torch.Tensor]) -> Optional[A.ConvTensor]:
    """Tensor descriptor (sizes, element strides, dtype) of a torch tensor."""
    if t is None:
        return None
    if t.dtype not in _TORCH_DT:
        raise TypeError(f"unsupported dtype {t.dtype}")
    if t.dim() > A.MAX_RANK:
        raise ValueError("at most 5 dims")
    d = A.ConvTensor()
    d.rank = t.dim()
    d.dtype = _TORCH_DT[t.dtype]
    for i, (s, st) in enumerate(zip(t.shape, t.stride())):
        d.sizes[i] = s
        d.strides[i] = st
    return d


def tensor_desc(sizes: Sequence[int], strides: Sequence[int], dtype: torch.dtype) -> A.ConvTensor:
    d = A.ConvTensor()
    d.rank = len(sizes)
    d.dtype = _TORCH_DT[dtype]
    for i, (s, st) in enumerate(zip(sizes, strides)):
        d.sizes[i] = s
        d.strides[i] = st
    return d


def _list(v) -> Tuple[int, ...]:
    if v is None:
        return ()
    if isinstance(v, int):
        return (v,)
    return tuple(int(a) for a in v)


def make_args(*, transposed: bool = False, groups: int = 1, stride=None, padding_before=None,
              padding_after=None, dilation=None, output_padding=None,
              padding_mode: str = "explicit") -> A.ConvArgs:
    a = A.ConvArgs()
    a.transposed = int(bool(transposed))
    a.padding_mode = {"explicit": A.PAD_EXPLICIT, "same": A.PAD_SAME, "valid": A.PAD_VALID}[padding_mode]
    a.groups = int(groups)
    pb, pa = _list(padding_before), _list(padding_after)
    if len(pb) != len(pa):
        raise ValueError("padding_before and padding_after need the same number of values")
    for name, vals in (("stride", _list(stride)), ("padding_before", pb), ("padding_after", pa),
                       ("dilation", _list(dilation)), ("output_padding", _list(output_padding))):
        if len(vals) > A.MAX_SPATIAL:
            raise ValueError(f"{name}: at most 3 values")
        arr = getattr(a, name)
        for i, v in enumerate(vals):
            arr[i] = v
    a.n_stride = len(_list(stride))
    a.n_padding = len(pb)
    a.n_dilation = len(_list(dilation))
    a.n_output_padding = len(_list(output_padding))
    return a


# ------------------------------------------------------------ the four calls --

def conv_bind(x: A.ConvTensor, w: A.ConvTensor, b: Optional[A.ConvTensor],
              args: A.ConvArgs) -> A.ConvDesc:
    d = A.ConvDesc()
    err = ctypes.create_string_buffer(256)
    st = A.lib().conv_bind(ctypes.byref(x), ctypes.byref(w), ctypes.byref(b) if b is not None else None,
                           ctypes.byref(args), ctypes.byref(d), err, len(err))
    _check(st, err.value.decode())
    return d


def conv_out_shape(d: A.ConvDesc) -> Tuple[Tuple[int, ...], Tuple[int, ...]]:
    y = A.ConvTensor()
    _check(A.lib().conv_out_shape(ctypes.byref(d), ctypes.byref(y)))
    return tuple(y.sizes[: y.rank]), tuple(y.strides[: y.rank])


def conv_plan(d: A.ConvDesc, y: A.ConvTensor, force_kernel: Union[int, str, None] = None,
              force_variant: Optional[int] = None) -> A.ConvPlan:
    """``conv_plan``, or ``conv_plan_ex`` when a schedule is forced too."""
    if force_kernel is None:
        force_kernel = "auto"
    if isinstance(force_kernel, str):
        force_kernel = A.KERNELS[force_kernel]
    p = A.ConvPlan()
    if force_variant is None:
        _check(A.lib().conv_plan(ctypes.byref(d), ctypes.byref(y), int(force_kernel), ctypes.byref(p)))
    else:
        o = A.ConvPlanOpts()
        o.force_kernel = int(force_kernel)
        o.force_variant = int(force_variant)
        _check(A.lib().conv_plan_ex(ctypes.byref(d), ctypes.byref(y), ctypes.byref(o), ctypes.byref(p)))
    return p


def conv_run(p: A.ConvPlan, x_ptr: int, w_ptr: int, b_ptr: Optional[int], y_ptr: int,
             ws_ptr: Optional[int] = None, ws_bytes: int = 0, stream: Optional[int] = None) -> None:
    _check(A.lib().conv_run(ctypes.byref(p), x_ptr, w_ptr, b_ptr, y_ptr, ws_ptr, ws_bytes, stream))


def conv_plan_candidates(d: A.ConvDesc, y: A.ConvTensor):
    """Every plan that can run the call (the rule's plan first)."""
    n = ctypes.c_int32(0)
    _check(A.lib().conv_plan_candidates(ctypes.byref(d), ctypes.byref(y), None, 0, ctypes.byref(n)))
    arr = (A.ConvPlan * max(1, n.value))()
    _check(A.lib().conv_plan_candidates(ctypes.byref(d), ctypes.byref(y), arr, n.value, ctypes.byref(n)))
    return list(arr[: n.value])


def conv_plan_tuned(d: A.ConvDesc, y: A.ConvTensor) -> A.ConvPlan:
    p = A.ConvPlan()
    _check(A.lib().conv_plan_tuned(ctypes.byref(d), ctypes.byref(y), ctypes.byref(p)))
    return p


def kernel_name(k: int) -> str:
    return A.lib().conv_kernel_name(k).decode()


# -------------------------------------------------------------- torch helper --

class Prepared:
    """bind + out_shape + plan for fixed tensor descriptors (reusable)."""

    def __init__(self, x: torch.Tensor, w: torch.Tensor, b: Optional[torch.Tensor], args: A.ConvArgs,
                 force_kernel=None, force_variant: Optional[int] = None, tuned: bool = False):
        self.desc = conv_bind(describe(x), describe(w), describe(b), args)
        self.sizes, self.strides = conv_out_shape(self.desc)
        self.dtype = x.dtype
        ydesc = tensor_desc(self.sizes, self.strides, x.dtype)
        if tuned and force_kernel is None and force_variant is None:
            self.plan = conv_plan_tuned(self.desc, ydesc)
        else:
            self.plan = conv_plan(self.desc, ydesc, force_kernel, force_variant)

    def empty_output(self, device) -> torch.Tensor:
        return torch.empty_strided(self.sizes, self.strides, dtype=self.dtype, device=device)

    def tune(self, x: torch.Tensor, w: torch.Tensor, b: Optional[torch.Tensor], reps: int = 5) -> A.ConvPlan:
        """Time every candidate schedule on these buffers (conv_tune) and keep
        the fastest; later Prepared(..., tuned=True) of the same descriptors
        on this device get it from the library's cache."""
        y = self.empty_output(x.device)
        ydesc = tensor_desc(self.sizes, self.strides, self.dtype)
        need = max(int(p.workspace_bytes) for p in conv_plan_candidates(self.desc, ydesc))
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
        best = A.ConvPlan()
        stream = torch.cuda.current_stream(x.device).cuda_stream
        _check(A.lib().conv_tune(ctypes.byref(self.desc), ctypes.byref(ydesc), x.data_ptr(), w.data_ptr(),
                                 b.data_ptr() if b is not None else None, y.data_ptr(), ws.data_ptr(), ws.numel(),
                                 stream, int(reps), ctypes.byref(best)))
        self.plan = best
        return best

    def workspace(self, device) -> Optional[torch.Tensor]:
        n = int(self.plan.workspace_bytes)
        return torch.empty(n, dtype=torch.uint8, device=device) if n else None

    def run(self, x: torch.Tensor, w: torch.Tensor, b: Optional[torch.Tensor], y: torch.Tensor,
            ws: Optional[torch.Tensor] = None, stream: Optional[int] = None) -> torch.Tensor:
        if stream is None:
            stream = torch.cuda.current_stream(x.device).cuda_stream
        conv_run(self.plan, x.data_ptr(), w.data_ptr(), b.data_ptr() if b is not None else None,
                 y.data_ptr(), ws.data_ptr() if ws is not None else None,
                 ws.numel() if ws is not None else 0, stream)
        return y


def conv(x: torch.Tensor, w: torch.Tensor, b: Optional[torch.Tensor] = None, *, stride=1,
         padding_before=0, padding_after=0, dilation=1, groups: int = 1, transposed: bool = False,
         output_padding=0, padding_mode: str = "explicit", force_kernel=None,
         force_variant: Optional[int] = None, tune: bool = False) -> torch.Tensor:
    """The canonical convolution on GPU tensors (x, w, b share one dtype).
    ``tune``: use the schedule conv_tune chose for these descriptors, timing
    the candidates first if they have not been timed on this device."""
    for t in (x, w) + ((b,) if b is not None else ()):
        if not t.is_cuda:
            raise ValueError("the canonical convolution runs on the GPU only; move tensors to cuda")
    if padding_mode != "explicit":
        padding_before = padding_after = None
    args = make_args(transposed=transposed, groups=groups, stride=stride,
                     padding_before=padding_before, padding_after=padding_after,
                     dilation=dilation, output_padding=output_padding if transposed else None,
                     padding_mode=padding_mode)
    prep = Prepared(x, w, b, args, force_kernel, force_variant, tuned=tune)
    if tune and force_kernel is None and force_variant is None and not (prep.plan.flags & A.PLAN_TUNED):
        prep.tune(x, w, b)
    y = prep.empty_output(x.device)
    return prep.run(x, w, b, y, prep.workspace(x.device))


# -------------------------------------------------------------- gradients --

def _tensor_of(d: A.ConvTensor):
    return tuple(d.sizes[: d.rank]), tuple(d.strides[: d.rank])


class PreparedBackward:
    """conv_plan_backward for fixed descriptors (reusable): the input, weight
    and bias gradients of one call (torch/_inductor/kernel/conv.py,
    convolution_backward)."""

    def __init__(self, x: torch.Tensor, w: torch.Tensor, gy: torch.Tensor, args: A.ConvArgs, *,
                 need_dx: bool = True, need_dw: bool = True, need_db: bool = True):
        self.desc = conv_bind(describe(x), describe(w), None, args)
        self.dtype = x.dtype
        gyd = describe(gy)
        self.plan = A.ConvBwdPlan()
        _check(A.lib().conv_plan_backward(ctypes.byref(self.desc), ctypes.byref(gyd), int(need_dx), int(need_dw),
                                          int(need_db), ctypes.byref(self.plan)))
        dx, dw, db = A.ConvTensor(), A.ConvTensor(), A.ConvTensor()
        _check(A.lib().conv_backward_layout(ctypes.byref(self.desc), ctypes.byref(gyd), ctypes.byref(dx) if need_dx
                                            else None, ctypes.byref(dw), ctypes.byref(db)))
        self.dx_layout = _tensor_of(dx) if need_dx else None
        self.dw_layout = _tensor_of(dw) if need_dw else None
        self.db_layout = _tensor_of(db) if need_db else None

    def outputs(self, device):
        mk = lambda lay: None if lay is None else torch.empty_strided(lay[0], lay[1], dtype=self.dtype, device=device)
        return mk(self.dx_layout), mk(self.dw_layout), mk(self.db_layout)

    def workspace(self, device) -> Optional[torch.Tensor]:
        n = int(self.plan.workspace_bytes)
        return torch.empty(n, dtype=torch.uint8, device=device) if n else None

    def run(self, x, w, gy, dx=None, dw=None, db=None, ws=None, stream: Optional[int] = None):
        if stream is None:
            stream = torch.cuda.current_stream(gy.device).cuda_stream
        ptr = lambda t: t.data_ptr() if t is not None else None
        _check(A.lib().conv_run_backward(ctypes.byref(self.plan), ptr(x), ptr(w), ptr(gy), ptr(dx), ptr(dw), ptr(db),
                                         ptr(ws), ws.numel() if ws is not None else 0, stream))
        return dx, dw, db


def conv_backward(x: torch.Tensor, w: torch.Tensor, gy: torch.Tensor, *, stride=1, padding_before=0,
                  padding_after=0, dilation=1, groups: int = 1, transposed: bool = False, output_padding=0,
                  padding_mode: str = "explicit", need_dx: bool = True, need_dw: bool = True,
                  need_db: bool = True):
    """Gradients (dx, dw, db) of the canonical convolution for an output
    gradient gy (GPU tensors; a gradient not asked for is None)."""
    for t in (x, w, gy):
        if not t.is_cuda:
            raise ValueError("the canonical convolution runs on the GPU only; move tensors to cuda")
    if padding_mode != "explicit":
        padding_before = padding_after = None
    args = make_args(transposed=transposed, groups=groups, stride=stride, padding_before=padding_before,
                     padding_after=padding_after, dilation=dilation,
                     output_padding=output_padding if transposed else None, padding_mode=padding_mode)
    prep = PreparedBackward(x, w, gy, args, need_dx=need_dx, need_dw=need_dw, need_db=need_db)
    dx, dw, db = prep.outputs(gy.device)
    return prep.run(x, w, gy, dx, dw, db, prep.workspace(gy.device))


# ------------------------------------------------------- ATen-style overloads --

def _pad_args(padding):
    if isinstance(padding, str):
        return dict(padding_mode=padding)
    p = _list(padding)
    return dict(padding_before=p, padding_after=p)


def conv1d(input, weight, bias=None, stride=1, padding=0, dilation=1, groups=1):
    return conv(input, weight, bias, stride=stride, dilation=dilation, groups=groups, **_pad_args(padding))


conv2d = conv1d
conv3d = conv1d


def conv_transpose1d(input, weight, bias=None, stride=1, padding=0, output_padding=0, groups=1,
                     dilation=1):
    p = _list(padding)
    return conv(input, weight, bias, stride=stride, padding_before=p, padding_after=p, dilation=dilation,
                groups=groups, transposed=True, output_padding=output_padding)


conv_transpose2d = conv_transpose1d
conv_transpose3d = conv_transpose1d


def convolution(input, weight, bias, stride, padding, dilation, transposed, output_padding, groups):
    """``aten.convolution``: symmetric padding, explicit transposed flag."""
    p = _list(padding)
    return conv(input, weight, bias, stride=stride, padding_before=p, padding_after=p, dilation=dilation,
                groups=groups, transposed=bool(transposed), output_padding=output_padding)


def _convolution(input, weight, bias, stride, padding, dilation, transposed, output_padding, groups,
                 benchmark=False, deterministic=False, cudnn_enabled=True, allow_tf32=True):
    """``aten._convolution``: the extra flags select nothing here (fp32 inputs
    are always computed in full fp32, never in a TF32-class mode)."""
    return convolution(input, weight, bias, stride, padding, dilation, transposed, output_padding, groups)
