"""Seeded synthetic inputs for the canonical convolution.

This module holds shapes, value distributions and seeds only -- none of the
convolution's arithmetic -- so both the GPU path's tests and the reference
checker can draw identical inputs from it.  It imports torch and nothing from
the rest of the package.

Generation recipe (identical for every workload):
  1. ``g = torch.Generator('cpu').manual_seed(seed)``.
  2. Draw float32 values in the order x, w, b, each in its logical
     [N, C, spatial...] / [C_out, C_in/groups, k...] order.
     U(a, b) is ``a + (b - a) * rand``; N(0, v) is ``sqrt(v) * randn`` (v is the
     variance).
  3. Cast to the workload dtype with ``.to(dtype)`` (round to nearest even).
  4. Apply the memory format (channels-last / NLC), then copy to the device.
The reference checker receives ``.double()`` of the same cast tensors.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Sequence, Tuple

import torch

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclasses.dataclass(frozen=True)
class Workload:
    """One convolution call with its synthetic-input recipe."""

    name: str
    x_shape: Tuple[int, ...]          # logical [N, C_in, L...]
    w_shape: Tuple[int, ...]          # [C_out, Cig, k...] or [C_in, Cog, k...] (transposed)
    dtype: str                        # "f32" | "f16" | "bf16"
    channels_last: bool               # x stored channels-last (NHWC / NLC)
    has_bias: bool
    groups: int = 1
    stride: Tuple[int, ...] = (1,)
    padding_before: Tuple[int, ...] = (0,)
    padding_after: Tuple[int, ...] = (0,)
    dilation: Tuple[int, ...] = (1,)
    transposed: bool = False
    output_padding: Tuple[int, ...] = (0,)
    x_dist: Tuple = ("normal", 1.0)   # ("uniform", a, b) | ("normal", variance)
    w_dist: Tuple = ("normal", 1.0)
    b_dist: Tuple = ("uniform", -0.1, 0.1)
    seed: int = 0

    def conv_kwargs(self) -> Dict:
        return dict(stride=self.stride, padding_before=self.padding_before,
                    padding_after=self.padding_after, dilation=self.dilation,
                    groups=self.groups, transposed=self.transposed,
                    output_padding=self.output_padding)

    def with_batch(self, n: int) -> "Workload":
        """Same call with a different batch size (same seed and recipe)."""
        return dataclasses.replace(self, name=f"{self.name}@N{n}",
                                   x_shape=(n,) + tuple(self.x_shape[1:]))


def _draw(g: torch.Generator, shape, dist) -> torch.Tensor:
    kind = dist[0]
    if kind == "uniform":
        a, b = float(dist[1]), float(dist[2])
        return a + (b - a) * torch.rand(shape, generator=g, dtype=torch.float32)
    if kind == "normal":
        return math.sqrt(float(dist[1])) * torch.randn(shape, generator=g, dtype=torch.float32)
    if kind == "ones":
        return torch.ones(shape, dtype=torch.float32)
    if kind == "ints":          # small integers in [lo, hi]
        lo, hi = int(dist[1]), int(dist[2])
        return torch.randint(lo, hi + 1, shape, generator=g).to(torch.float32)
    raise ValueError(f"unknown distribution {dist}")


def channels_last_copy(t: torch.Tensor) -> torch.Tensor:
    """Dense copy with the channel dim fastest (NLC / NHWC / NDHWC)."""
    nd = t.dim()
    perm = [0] + list(range(2, nd)) + [1]
    inv = [0] * nd
    for i, p in enumerate(perm):
        inv[p] = i
    return t.permute(perm).contiguous().permute(inv)


def make_inputs(wl: Workload, device: Optional[str] = None):
    """Return (x, w, b) for a workload: cast, laid out, on ``device``."""
    g = torch.Generator("cpu").manual_seed(int(wl.seed))
    x = _draw(g, wl.x_shape, wl.x_dist)
    w = _draw(g, wl.w_shape, wl.w_dist)
    c_out = wl.w_shape[1] * wl.groups if wl.transposed else wl.w_shape[0]
    b = _draw(g, (c_out,), wl.b_dist) if wl.has_bias else None
    dt = DTYPES[wl.dtype]
    x, w = x.to(dt), w.to(dt)
    b = b.to(dt) if b is not None else None
    if wl.channels_last:
        x = channels_last_copy(x)
    if device is not None:
        x = x.to(device)
        w = w.to(device)
        b = b.to(device) if b is not None else None
    return x, w, b


# --- The five measured workloads -------------------------------------------

def depthwise_f32_small() -> Workload:
    """Depthwise 3x3, fp32 NCHW, N=1, C=32, 32x32, pad 1/1, bias."""
    return Workload("dw_f32_nchw_1x32x32x32_k3", (1, 32, 32, 32), (32, 1, 3, 3), "f32", False,
                    True, groups=32, stride=(1, 1), padding_before=(1, 1), padding_after=(1, 1),
                    dilation=(1, 1), output_padding=(0, 0), x_dist=("uniform", -1.0, 1.0),
                    w_dist=("uniform", -1.0, 1.0), b_dist=("uniform", -0.1, 0.1), seed=1)


def depthwise_bf16_cl(k: int, s: int) -> Workload:
    """Depthwise k x k, bf16 channels-last, N=32, C=256, 56x56, bias.

    stride 1: symmetric 'same' padding k//2 on both sides;
    stride 2: padding_before = k//2 - 1, padding_after = k//2."""
    if s == 1:
        pb, pa = k // 2, k // 2
    else:
        pb, pa = k // 2 - 1, k // 2
    return Workload(f"dw_bf16_nhwc_32x256x56x56_k{k}s{s}", (32, 256, 56, 56), (256, 1, k, k),
                    "bf16", True, True, groups=256, stride=(s, s), padding_before=(pb, pb),
                    padding_after=(pa, pa), dilation=(1, 1), output_padding=(0, 0),
                    x_dist=("normal", 1.0), w_dist=("normal", 1.0 / (k * k)),
                    b_dist=("uniform", -0.1, 0.1), seed=2000 + 10 * k + s)


def depthwise_bf16_cl_all() -> List[Workload]:
    return [depthwise_bf16_cl(k, s) for k in (3, 5, 7) for s in (1, 2)]


def grouped_f16() -> Workload:
    """Grouped 3x3, fp16 NCHW, N=32, 256 -> 512 channels, 64 groups, 28x28."""
    return Workload("grp_f16_nchw_32x256x28x28_g64_m2", (32, 256, 28, 28), (512, 4, 3, 3), "f16",
                    False, False, groups=64, stride=(1, 1), padding_before=(1, 1),
                    padding_after=(1, 1), dilation=(1, 1), output_padding=(0, 0),
                    x_dist=("normal", 1.0), w_dist=("normal", 1.0 / 36.0), seed=3)


def dense_bf16_cl() -> Workload:
    """Dense 3x3, bf16 channels-last, N=64, 256 -> 256 channels, 56x56, bias."""
    return Workload("dense_bf16_nhwc_64x256x56x56_k3", (64, 256, 56, 56), (256, 256, 3, 3),
                    "bf16", True, True, groups=1, stride=(1, 1), padding_before=(1, 1),
                    padding_after=(1, 1), dilation=(1, 1), output_padding=(0, 0),
                    x_dist=("normal", 1.0), w_dist=("normal", 1.0 / 2304.0),
                    b_dist=("uniform", -0.1, 0.1), seed=4)


def transposed_bf16_nlc() -> Workload:
    """Transposed 1-D, bf16 NLC, N=16, 512 -> 512 channels, L 8192, k=4, s=2,
    padding_before=1, padding_after=2, output_padding=0, no bias."""
    return Workload("convT1d_bf16_nlc_16x512x8192_k4s2", (16, 512, 8192), (512, 512, 4), "bf16",
                    True, False, groups=1, stride=(2,), padding_before=(1,), padding_after=(2,),
                    dilation=(1,), transposed=True, output_padding=(0,),
                    x_dist=("normal", 1.0), w_dist=("normal", 1.0 / 2048.0), seed=5)


# --- Calls at the edges of the fast paths (measured, not part of the five) --

def domain_edge_workloads() -> List[Workload]:
    """Calls of the canonical domain outside the five measured workloads, with
    the channel and spatial sizes of the depthwise workload where they apply:
    depthwise 9x9 and stride 3, a channel multiplier of 2, 1-D depthwise
    (NLC), 3-D dense forward and 2-D transposed (channels-last), and grouped
    1-D transposed with dilation 2."""
    out = []
    def dw(name, x, w, groups, k, s, pb, pa, seed):
        r = len(k)
        taps = 1
        for v in k:
            taps *= v
        return Workload(name, x, w, "bf16", True, True, groups=groups, stride=s, padding_before=pb,
                        padding_after=pa, dilation=(1,) * r, output_padding=(0,) * r,
                        x_dist=("normal", 1.0), w_dist=("normal", 1.0 / taps), b_dist=("uniform", -0.1, 0.1),
                        seed=seed)
    out.append(dw("edge_dw_bf16_nhwc_32x256x56x56_k9s1", (32, 256, 56, 56), (256, 1, 9, 9), 256, (9, 9), (1, 1),
                  (4, 4), (4, 4), 3001))
    out.append(dw("edge_dw_bf16_nhwc_32x256x56x56_k3s3", (32, 256, 56, 56), (256, 1, 3, 3), 256, (3, 3), (3, 3),
                  (1, 1), (1, 1), 3002))
    out.append(dw("edge_dw_bf16_nhwc_32x256x56x56_k3s1_m2", (32, 256, 56, 56), (512, 1, 3, 3), 256, (3, 3), (1, 1),
                  (1, 1), (1, 1), 3003))
    out.append(Workload("edge_dw1d_bf16_nlc_32x256x3136_k7", (32, 256, 3136), (256, 1, 7), "bf16", True, True,
                        groups=256, stride=(1,), padding_before=(3,), padding_after=(3,), dilation=(1,),
                        output_padding=(0,), x_dist=("normal", 1.0), w_dist=("normal", 1.0 / 7.0),
                        b_dist=("uniform", -0.1, 0.1), seed=3004))
    out.append(Workload("edge_dense3d_bf16_ndhwc_4x128x16x28x28_k3", (4, 128, 16, 28, 28), (128, 128, 3, 3, 3),
                        "bf16", True, True, groups=1, stride=(1, 1, 1), padding_before=(1, 1, 1),
                        padding_after=(1, 1, 1), dilation=(1, 1, 1), output_padding=(0, 0, 0),
                        x_dist=("normal", 1.0), w_dist=("normal", 1.0 / 3456.0), b_dist=("uniform", -0.1, 0.1),
                        seed=3005))
    out.append(Workload("edge_convT2d_bf16_nhwc_16x256x28x28_k4s2", (16, 256, 28, 28), (256, 128, 4, 4), "bf16",
                        True, True, groups=1, stride=(2, 2), padding_before=(1, 1), padding_after=(1, 1),
                        dilation=(1, 1), transposed=True, output_padding=(0, 0), x_dist=("normal", 1.0),
                        w_dist=("normal", 1.0 / 1024.0), b_dist=("uniform", -0.1, 0.1), seed=3006))
    return out


def all_workloads() -> List[Workload]:
    return ([depthwise_f32_small()] + depthwise_bf16_cl_all()
            + [grouped_f16(), dense_bf16_cl(), transposed_bf16_nlc()])


def random_case(seed: int, *, rank: int, transposed: bool, dtype: str, channels_last: bool,
                N: int, C_in: int, C_out: int, groups: int, L: Sequence[int], k: Sequence[int],
                stride: Sequence[int], padding_before: Sequence[int], padding_after: Sequence[int],
                dilation: Sequence[int], output_padding: Sequence[int], has_bias: bool,
                x_dist=("normal", 1.0), w_dist=None, b_dist=("uniform", -0.5, 0.5)) -> Workload:
    """A workload for parity sweeps (weights scaled by fan-in unless given)."""
    cig = C_in // groups
    taps = 1
    for kk in k:
        taps *= kk
    if w_dist is None:
        w_dist = ("normal", 1.0 / max(1, cig * taps))
    if transposed:
        w_shape = (C_in, C_out // groups) + tuple(k)
    else:
        w_shape = (C_out, cig) + tuple(k)
    return Workload(f"case{seed}", (N, C_in) + tuple(L), w_shape, dtype, channels_last, has_bias,
                    groups=groups, stride=tuple(stride), padding_before=tuple(padding_before),
                    padding_after=tuple(padding_after), dilation=tuple(dilation),
                    transposed=transposed, output_padding=tuple(output_padding),
                    x_dist=x_dist, w_dist=w_dist, b_dist=b_dist, seed=seed)
