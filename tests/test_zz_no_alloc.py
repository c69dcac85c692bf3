"""delta_fwd_noalloc (the entry point that allocates nothing) against delta_fwd:
two calls in a row on one GPU, the second with a smaller input, each compared
with delta_fwd on the same inputs (the same kernels, so bitwise equal), for the
forms that use the scratch and one that does not."""
import numpy as np
import pytest
import torch

from gpu_util import announce, dev
from recurrent_memory_amd import ops
from recurrent_memory_amd.inputs import Workload, make_forward_inputs

pytestmark = pytest.mark.gpu


def _both(variant, dtype, w):
    x = make_forward_inputs(w)
    t = {n: dev(a, "f32" if n == "S0" else dtype) for n, a in x.items()}
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    o_ref, S_ref = ops.delta_fwd(variant, t["q"], t["k"], t["v"], t["beta"], wgate=t["wgate"], g=t["g"], S0=t["S0"])
    o = torch.full((w.B, w.T, w.H, w.dv), float("nan"), dtype=tdt, device="cuda")
    S = torch.full((w.B, w.H, w.dv, w.dk), float("nan"), dtype=torch.float32, device="cuda")
    ops.delta_fwd_noalloc(variant, t["q"], t["k"], t["v"], t["beta"], o, wgate=t["wgate"], g=t["g"], S0=t["S0"], S_T=S)
    torch.cuda.synchronize()
    return o, S, o_ref, S_ref


@pytest.mark.parametrize("variant,dtype", [("kda", "bf16"), ("gdn2", "bf16"), ("fg2", "bf16"), ("gdn", "bf16")])
def test_noalloc_matches_delta_fwd_twice(variant, dtype):
    for i, (B, H, T) in enumerate([(2, 8, 1000), (1, 3, 77)]):   # the second call is smaller
        announce("noalloc", variant, dtype, B, H, T)
        w = Workload("t", variant, dtype, B=B, H=H, T=T, dk=128, dv=128, random_s0=True, seed=120 + i)
        o, S, o_ref, S_ref = _both(variant, dtype, w)
        assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)), (variant, i)
        assert torch.equal(S, S_ref), (variant, i)


def test_noalloc_rejects_workloads_beyond_its_scratch():
    """KDA bf16 at B*H*ceil(T/32) = 1725 blocks of 38 KiB needs more than 64 MiB."""
    desc = ops.DrDesc(1, 1725 * 32, 1, 128, 128, 64, ops.VARIANTS["kda"], 1, 1)
    assert ops.workspace_bytes("fwd", desc) > 64 << 20
    B, T, H = 1, 1725 * 32, 1
    bf = torch.bfloat16
    q = torch.zeros((B, T, H, 128), dtype=bf, device="cuda")
    g = torch.zeros((B, T, H, 128), dtype=bf, device="cuda")
    o = torch.empty((B, T, H, 128), dtype=bf, device="cuda")
    with pytest.raises(ops.DeltaRuleError) as e:
        ops.delta_fwd_noalloc("kda", q, q.clone(), q.clone(), torch.zeros((B, T, H), dtype=bf, device="cuda"), o, g=g)
    assert e.value.status == 8
