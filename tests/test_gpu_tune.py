"""Plan-time schedule timing (conv_tune / conv_plan_tuned) on the GPU: the
chosen plan is one of the candidates, it is cached per descriptor, and the
calls it runs match the reference."""
import pytest
import torch

import oracle
from depthwise_stencil_implicit_amd import _abi as A
from depthwise_stencil_implicit_amd import api, synth

from gpu_util import EPS, assert_close, expand_kw, ref_inputs

pytestmark = pytest.mark.gpu

CASES = [
    synth.dense_bf16_cl().with_batch(2),
    synth.transposed_bf16_nlc().with_batch(1),
    synth.depthwise_bf16_cl(7, 1).with_batch(2),
    synth.grouped_f16().with_batch(2),
    synth.depthwise_f32_small(),
]


def _args(wl):
    kw = expand_kw(wl)
    return api.make_args(**{k: v for k, v in kw.items() if k not in ("groups", "transposed")}, groups=wl.groups,
                         transposed=wl.transposed)


@pytest.mark.parametrize("wl", CASES, ids=lambda w: w.name)
def test_tuned_plan_is_cached_and_correct(wl):
    print(f"tune: {wl.name}", flush=True)
    x, w, b = synth.make_inputs(wl, device="cuda")
    prep = api.Prepared(x, w, b, _args(wl))
    cands = api.conv_plan_candidates(prep.desc, api.tensor_desc(prep.sizes, prep.strides, x.dtype))
    best = prep.tune(x, w, b, reps=3)
    keys = {(int(c.kernel), int(c.variant), int(c.flags)) for c in cands}
    assert (int(best.kernel), int(best.variant), int(best.flags)) in keys
    print(f"  chose {api.kernel_name(best.kernel)} variant {best.variant} of {len(cands)} candidates", flush=True)
    again = api.Prepared(x, w, b, _args(wl), tuned=True)
    assert again.plan.flags & A.PLAN_TUNED
    assert (again.plan.kernel, again.plan.variant) == (best.kernel, best.variant)
    y = again.run(x, w, b, again.empty_output(x.device), again.workspace(x.device))
    torch.cuda.synchronize()
    yr, Ar = oracle.conv(*ref_inputs(x, w, b), **expand_kw(wl))
    assert_close(y, yr, Ar, EPS[wl.dtype], f"{wl.name} tuned")


def test_conv_tune_flag_runs_the_tuned_schedule():
    wl = synth.random_case(9300, rank=2, transposed=False, dtype="f16", channels_last=True, N=2, C_in=64,
                           C_out=96, groups=1, L=[17, 19], k=[3, 3], stride=[1, 1], padding_before=[1, 1],
                           padding_after=[1, 1], dilation=[1, 1], output_padding=[0, 0], has_bias=True)
    x, w, b = synth.make_inputs(wl, device="cuda")
    kw = expand_kw(wl)
    y = api.conv(x, w, b, stride=kw["stride"], padding_before=kw["padding_before"],
                 padding_after=kw["padding_after"], tune=True)
    torch.cuda.synchronize()
    yr, Ar = oracle.conv(*ref_inputs(x, w, b), **kw)
    assert_close(y, yr, Ar, EPS["f16"], "conv(tune=True)")
    assert api.Prepared(x, w, b, _args(wl), tuned=True).plan.flags & A.PLAN_TUNED
