"""Decode step on the GPU against the oracle's decode step."""
import numpy as np
import pytest
import torch

from gpu_util import LOG_DECAY_FLOOR, TOL, announce, dev, host, slice_rel_err
from oracle import delta_decode as oracle_decode
from recurrent_memory_amd import ops
from recurrent_memory_amd.inputs import WORKLOADS, Workload, make_decode_inputs

pytestmark = pytest.mark.gpu


def _run_steps(variant, dtype, d, n_steps, pool=None):
    """Run n_steps GPU decode steps; step i uses input set i % len(steps)."""
    S = dev(d["S"], "f32")
    steps = [{n: dev(a, dtype) for n, a in s.items()} for s in d["steps"]]
    outs = []
    for i in range(n_steps):
        s = steps[i % len(steps)]
        o = ops.delta_decode(variant, s["q"], s["k"], s["v"], s["beta"], S, wgate=s["wgate"], g=s["g"])
        outs.append(o)
    torch.cuda.synchronize()
    return [host(o) for o in outs], host(S)


def _oracle_steps(variant, d, n_steps, heads=None):
    S = d["S"].astype(np.float64)
    sel = (lambda a: a) if heads is None else (lambda a: a[heads[0], heads[1]][:, None])
    S = sel(S) if heads is not None else S
    outs = []
    for i in range(n_steps):
        s = d["steps"][i % len(d["steps"])]
        args = {n: (None if a is None else sel(a)) for n, a in s.items()}
        o, S = oracle_decode(variant, **args, S=S)
        outs.append(o)
    return outs, S


@pytest.mark.parametrize("variant", ["deltanet", "gdn", "kda", "gdn2", "fg2"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 128), (128, 64), (64, 64)])
def test_decode_small(variant, dtype, dk, dv):
    announce("decode_small", variant, dtype, dk, dv)
    w = Workload("t", variant, dtype, B=3, H=5, T=1, dk=dk, dv=dv, random_s0=True, seed=11)
    d = make_decode_inputs(w, 4)
    outs, S = _run_steps(variant, dtype, d, 4)
    ref_outs, S_ref = _oracle_steps(variant, d, 4)
    for o, r in zip(outs, ref_outs):
        assert slice_rel_err(o, r, (0, 1)) <= TOL[dtype]
    assert slice_rel_err(S, S_ref, (0, 1)) <= 1e-5


@pytest.mark.parametrize("variant", ["kda", "gdn2", "fg2"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_gate_floor(variant, dtype):
    """Channel log-decays of -10 are clamped to -85/16 on load, as in the forward,
    so decode continues a prefill on the same gates: equal to the oracle on the
    clamped gates."""
    announce("decode_gate_floor", variant, dtype)
    w = Workload("t", variant, dtype, B=3, H=5, T=1, dk=128, dv=128, random_s0=True, seed=12)
    d = make_decode_inputs(w, 3)
    for i, st in enumerate(d["steps"]):
        g = st["g"].copy()
        g[..., 3] = -10.0
        if i == 1:
            g[...] = -10.0
        st["g"] = g
    outs, S = _run_steps(variant, dtype, d, 3)
    for st in d["steps"]:
        st["g"] = np.maximum(st["g"], LOG_DECAY_FLOOR)
    ref_outs, S_ref = _oracle_steps(variant, d, 3)
    for o, r in zip(outs, ref_outs):
        assert slice_rel_err(o, r, (0, 1)) <= TOL[dtype]
    assert slice_rel_err(S, S_ref, (0, 1)) <= 1e-5


def test_decode_full_size_all_heads_three_steps():
    w = WORKLOADS["gdn_decode_bf16_b256_h16_d128"]
    announce("decode_full_all_heads", w.name)
    d = make_decode_inputs(w, 3)
    outs, S = _run_steps("gdn", "bf16", d, 3)
    ref_outs, S_ref = _oracle_steps("gdn", d, 3)
    for o, r in zip(outs, ref_outs):
        assert slice_rel_err(o, r, (0, 1)) <= TOL["bf16"]
    assert slice_rel_err(S, S_ref, (0, 1)) <= 1e-5


def test_decode_full_size_thousand_steps_sampled_heads():
    """1000 successive steps on the full 256 x 16 state; 16 fixed (batch, head)
    states checked against the oracle (step inputs cycle over 8 drawn sets)."""
    w = WORKLOADS["gdn_decode_bf16_b256_h16_d128"]
    announce("decode_full_1000_steps", w.name)
    d = make_decode_inputs(w, 8)
    rng = np.random.default_rng(0)
    bs = rng.integers(0, w.B, 16)
    hs = rng.integers(0, w.H, 16)
    outs, S = _run_steps("gdn", "bf16", d, 1000)
    ref_outs, S_ref = _oracle_steps("gdn", d, 1000, heads=(bs, hs))
    for i in (0, 1, 500, 999):
        assert slice_rel_err(outs[i][bs, hs], ref_outs[i][:, 0], (0,)) <= TOL["bf16"]
    assert slice_rel_err(S[bs, hs], S_ref[:, 0], (0,)) <= 1e-4


@pytest.mark.parametrize("variant", ["kda", "gdn2", "fg2"])
def test_decode_full_size_channel_forms(variant):
    """The decode batch (256 x 16 heads, d = 128, bf16) for the channel-decay forms:
    3 steps, every head against the oracle."""
    import dataclasses
    w = dataclasses.replace(WORKLOADS["gdn_decode_bf16_b256_h16_d128"], variant=variant)
    announce("decode_full_channel", variant)
    d = make_decode_inputs(w, 3)
    outs, S = _run_steps(variant, "bf16", d, 3)
    ref_outs, S_ref = _oracle_steps(variant, d, 3)
    for o, r in zip(outs, ref_outs):
        assert slice_rel_err(o, r, (0, 1)) <= TOL["bf16"]
    assert slice_rel_err(S, S_ref, (0, 1)) <= 1e-5
