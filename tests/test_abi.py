"""The C-ABI library: it loads, exports every symbol the header declares, and
its struct layouts agree with the ctypes mirror (no GPU needed)."""
import ctypes
import os
import re
import subprocess

import pytest

from depthwise_stencil_implicit_amd import _abi as A

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "miconv.h")


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"MICONV_API\s+[\w\s\*]*?\b(conv_\w+)\s*\(", text)))


def test_header_declares_the_abi():
    assert declared_functions() == sorted(A.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = A.lib()
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", A.LIB_PATH], capture_output=True, text=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    assert set(declared_functions()) <= exported
    # Nothing but the C ABI is exported from the library's own code.
    assert {s for s in exported if s.startswith("conv_")} == set(declared_functions())


def test_abi_version_and_names():
    lib = A.lib()
    assert lib.conv_abi_version() == 3
    for name, val in A.KERNELS.items():
        assert lib.conv_kernel_name(val).decode() == name
    assert lib.conv_kernel_name(99).decode() == "?"
    assert lib.conv_status_string(A.ELAYOUT).decode().startswith("output layout")


PROBE = r"""
#include <stddef.h>
#include <stdio.h>
#include "miconv.h"
#define P(T, F) printf(#T "." #F " %zu\n", offsetof(T, F))
int main(void) {
  printf("conv_tensor %zu\nconv_args %zu\nconv_desc %zu\nconv_plan_t %zu\nconv_plan_opts %zu\n",
         sizeof(conv_tensor), sizeof(conv_args), sizeof(conv_desc), sizeof(conv_plan_t),
         sizeof(conv_plan_opts));
  P(conv_plan_opts, force_variant); P(conv_plan_opts, reserved);
  printf("conv_bwd_plan_t %zu\n", sizeof(conv_bwd_plan_t));
  P(conv_bwd_plan_t, gy); P(conv_bwd_plan_t, need_dx); P(conv_bwd_plan_t, dgrad); P(conv_bwd_plan_t, wg_tile);
  P(conv_bwd_plan_t, workspace_bytes); P(conv_bwd_plan_t, bytes);
  P(conv_args, groups); P(conv_args, stride); P(conv_args, output_padding);
  P(conv_desc, N); P(conv_desc, in); P(conv_desc, output_padding); P(conv_desc, x); P(conv_desc, b);
  P(conv_plan_t, y); P(conv_plan_t, kernel); P(conv_plan_t, workspace_bytes); P(conv_plan_t, tile);
  P(conv_plan_t, grid); P(conv_plan_t, block); P(conv_plan_t, flags); P(conv_plan_t, flops); P(conv_plan_t, bytes);
  return 0;
}
"""


def test_struct_layout_matches_ctypes(tmp_path):
    src = tmp_path / "probe.c"
    src.write_text(PROBE)
    exe = tmp_path / "probe"
    subprocess.check_call(["gcc", "-std=c99", f"-I{os.path.dirname(HEADER)}", str(src), "-o", str(exe)])
    got = dict(ln.rsplit(" ", 1) for ln in subprocess.check_output([str(exe)], text=True).splitlines())
    expect = {"conv_tensor": ctypes.sizeof(A.ConvTensor), "conv_args": ctypes.sizeof(A.ConvArgs),
              "conv_desc": ctypes.sizeof(A.ConvDesc), "conv_plan_t": ctypes.sizeof(A.ConvPlan),
              "conv_plan_opts": ctypes.sizeof(A.ConvPlanOpts), "conv_bwd_plan_t": ctypes.sizeof(A.ConvBwdPlan)}
    fields = {"conv_args": A.ConvArgs, "conv_desc": A.ConvDesc, "conv_plan_t": A.ConvPlan,
              "conv_plan_opts": A.ConvPlanOpts, "conv_bwd_plan_t": A.ConvBwdPlan}
    for key, val in got.items():
        if "." in key:
            struct, field = key.split(".")
            field = "in_" if field == "in" else field
            assert getattr(fields[struct], field).offset == int(val), key
        else:
            assert expect[key] == int(val), key
