"""DeltaTTT-pre on the GPU (delta_ttt_pre) against the oracle's ttt_pre_fwd."""
import numpy as np
import pytest
import torch

from oracle_pool import ttt_all_heads
from gpu_util import TOL, announce, dev, host, slice_rel_err
from oracle import ttt_pre_fwd
from recurrent_memory_amd import ops
from recurrent_memory_amd.inputs import Workload, make_ttt_inputs

pytestmark = pytest.mark.gpu


def _run(variant, dtype, x, in_place=False):
    A0 = dev(x["A0"], "f32") if x["A0"] is not None else None
    B0 = dev(x["B0"], "f32") if x["B0"] is not None else None
    kw = dict(A_T=A0, B_T=B0) if in_place else {}
    o, A_T, B_T = ops.ttt_pre(variant, dev(x["q"], dtype), dev(x["k"], dtype), dev(x["v"], dtype),
                              dev(x["beta1"], dtype), dev(x["beta2"], dtype), g1=dev(x["g1"], dtype),
                              g2=dev(x["g2"], dtype), A0=A0, B0=B0, **kw)
    torch.cuda.synchronize()
    return host(o), host(A_T), host(B_T)


def out_err(o, o_ref, v, dtype):
    """Per (batch, head) slice: max|o - o_ref| / max|o_ref|, the metric of every
    other parity test (bf16 inputs run through the fp32 path; only o is rounded)."""
    return slice_rel_err(o, o_ref, (0, 2))


def _check(variant, dtype, x, got):
    ref = ttt_pre_fwd(variant, x["q"], x["k"], x["v"], x["beta1"], x["g1"], x["beta2"], x["g2"],
                      x["A0"], x["B0"])
    errs = (out_err(got[0], ref[0], x["v"], dtype), slice_rel_err(got[1], ref[1], (0, 1)),
            slice_rel_err(got[2], ref[2], (0, 1)))
    assert max(errs) <= TOL[dtype], errs


@pytest.mark.parametrize("variant", ["deltanet", "gdn"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128), (128, 64), (64, 128)])
@pytest.mark.parametrize("T", [1, 65, 200])
def test_ttt_small(variant, dtype, dk, dv, T):
    announce("ttt_small", variant, dtype, dk, dv, T)
    w = Workload("t", variant, dtype, B=2, H=3, T=T, dk=dk, dv=dv, seed=60 + T + dk)
    x = make_ttt_inputs(w)
    _check(variant, dtype, x, _run(variant, dtype, x))


@pytest.mark.parametrize("variant", ["deltanet", "gdn"])
def test_ttt_zero_states_and_in_place(variant):
    announce("ttt_states", variant)
    w = Workload("t", variant, "f32", B=1, H=2, T=130, dk=128, dv=128, seed=70)
    x = make_ttt_inputs(w, random_states=False)
    o, A_T, B_T = _run(variant, "f32", x)
    _check(variant, "f32", x, (o, A_T, B_T))
    x = make_ttt_inputs(w)
    _check(variant, "f32", x, _run(variant, "f32", x, in_place=True))


def test_ttt_full_size_all_heads():
    """The headline shape (GDN, bf16, B=4 H=16 T=4096 d=128) through both layers;
    every (batch, head) sequence checked against the oracle end to end."""
    announce("ttt_full")
    w = Workload("t", "gdn", "bf16", B=4, H=16, T=4096, dk=128, dv=128, seed=71)
    x = make_ttt_inputs(w)
    got = _run("gdn", "bf16", x)
    ref = ttt_all_heads("gdn", x, w.B, w.H)
    errs = (out_err(got[0], ref[0], x["v"], "bf16"), slice_rel_err(got[1], ref[1], (0, 1)),
            slice_rel_err(got[2], ref[2], (0, 1)))
    assert max(errs) <= TOL["bf16"], errs
