"""Failure propagation on the GPU: a non-finite value in one (batch, head)
sequence never leaks into another sequence or into another value channel (value
rows of the memory are independent), leaves everything before its 64-token chunk
exactly as in a clean run, and makes every later output of its channel and its
row of the final state non-finite (it is not silently absorbed)."""
import numpy as np
import pytest
import torch

from gpu_util import announce, dev, host
from recurrent_memory_amd import ops
from recurrent_memory_amd.inputs import Workload, make_forward_inputs

pytestmark = pytest.mark.gpu


def _fwd(variant, dtype, x):
    o, S = ops.delta_fwd(variant, dev(x["q"], dtype), dev(x["k"], dtype), dev(x["v"], dtype),
                         dev(x["beta"], dtype), wgate=dev(x["wgate"], dtype), g=dev(x["g"], dtype),
                         S0=dev(x["S0"], "f32"))
    torch.cuda.synchronize()
    return host(o), host(S)


@pytest.mark.parametrize("variant", ["deltanet", "gdn", "kda", "gdn2", "fg2"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("bad", [np.nan, np.inf])
def test_non_finite_value_stays_in_its_sequence(variant, dtype, bad):
    announce("non_finite", variant, dtype, bad)
    w = Workload("t", variant, dtype, B=2, H=3, T=200, dk=128, dv=128, random_s0=True, seed=80)
    x = make_forward_inputs(w)
    o0, S0 = _fwd(variant, dtype, x)
    b, h, t = 1, 2, 137
    v = x["v"].copy()
    v[b, t, h, 5] = bad                                           # value channel 5
    o1, S1 = _fwd(variant, dtype, {**x, "v": v})
    others = np.ones((w.B, w.H), bool)
    others[b, h] = False
    assert np.array_equal(o1.transpose(0, 2, 1, 3)[others], o0.transpose(0, 2, 1, 3)[others])
    assert np.array_equal(S1[others], S0[others])
    c0 = (t // 64) * 64
    col = 5
    rest = [c for c in range(w.dv) if c != col]
    assert np.array_equal(o1[b, :, h][:, rest], o0[b, :, h][:, rest])   # other value channels
    assert np.array_equal(S1[b, h][rest], S0[b, h][rest])
    assert np.array_equal(o1[b, :c0, h], o0[b, :c0, h])          # earlier chunks untouched
    assert not np.isfinite(o1[b, t:, h, col]).any()               # every later output of the channel
    assert not np.isfinite(S1[b, h, col]).any()                   # and its row of the final state


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_non_finite_state_row_in_decode(dtype):
    """Decode works row by row: a NaN in one state matrix poisons that head's
    output and state only."""
    announce("non_finite_decode", dtype)
    from recurrent_memory_amd.inputs import make_decode_inputs
    w = Workload("t", "gdn", dtype, B=4, H=2, T=1, dk=128, dv=128, random_s0=True, seed=81)
    d = make_decode_inputs(w, 1)
    st = d["steps"][0]
    S_clean = d["S"].copy()
    S_bad = d["S"].copy()
    S_bad[2, 1, 7, 9] = np.nan
    outs = []
    for Sa in (S_clean, S_bad):
        S = torch.from_numpy(Sa).cuda()
        o = ops.delta_decode("gdn", *(dev(st[n], dtype) for n in ("q", "k", "v", "beta")), S, g=dev(st["g"], dtype))
        torch.cuda.synchronize()
        outs.append((host(o), host(S)))
    (oc, Sc), (ob, Sb) = outs
    mask = np.ones((w.B, w.H), bool)
    mask[2, 1] = False
    assert np.array_equal(ob[mask], oc[mask]) and np.array_equal(Sb[mask], Sc[mask])
    assert not np.isfinite(ob[2, 1]).all()
    assert np.isnan(Sb[2, 1, 7]).all()                            # the row that held the NaN
