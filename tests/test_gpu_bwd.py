"""Backward pass on the GPU (delta_bwd) against the oracle's reverse mode.

Every gradient of DeltaNet, GDN, KDA and GDN-2 in fp32 and bf16, at every head width,
for sequence lengths 1, 63, 64, 65 and 200 (ragged last chunk), with a random
initial state and a gradient arriving at the final state; plus a case with no
final-state gradient and dS0 not requested, and larger cases (T = 1024, 330 heads,
the timed GDN backward's full size) with every head checked.
"""
import numpy as np
import pytest
import torch

from oracle_pool import bwd_all_heads
from gpu_util import LOG_DECAY_FLOOR, TOL, announce, dev, floor_gates, host, slice_rel_err
from oracle import delta_bwd as oracle_bwd
from recurrent_memory_amd import ops
from recurrent_memory_amd.inputs import WORKLOADS, Workload, make_forward_inputs

pytestmark = pytest.mark.gpu

VARS = ["deltanet", "gdn", "kda", "gdn2", "fg2"]


def _upstream(w, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    dO = rng.standard_normal((w.B, w.T, w.H, w.dv), dtype=np.float32)
    dST = (0.5 * rng.standard_normal((w.B, w.H, w.dv, w.dk), dtype=np.float32)).astype(np.float32)
    if w.dtype == "bf16":
        from recurrent_memory_amd.inputs import round_to_bf16
        dO = round_to_bf16(dO)
    return dO, dST


def _run(variant, dtype, w, x, dO, dST, want_dS0=True):
    gr = ops.delta_bwd(variant, dev(x["q"], dtype), dev(x["k"], dtype), dev(x["v"], dtype),
                       dev(x["beta"], dtype), dev(dO, dtype), g=dev(x["g"], dtype),
                       S0=dev(x["S0"], "f32"), dS_T=dev(dST, "f32"), wgate=dev(x["wgate"], dtype),
                       want_dS0=want_dS0)
    torch.cuda.synchronize()
    return {n: host(t) for n, t in gr.items()}


def _check(variant, dtype, gr, ref, heads_axes=(0, 2)):
    tol = TOL[dtype]
    errs = {}
    for n in ("dq", "dk", "dv"):
        errs[n] = slice_rel_err(gr[n], ref[n], heads_axes)
    errs["dbeta"] = slice_rel_err(gr["dbeta"], ref["dbeta"], heads_axes)
    if variant == "gdn2":
        errs["dwgate"] = slice_rel_err(gr["dwgate"], ref["dwgate"], heads_axes)
    if variant != "deltanet":
        errs["dg"] = slice_rel_err(gr["dg"], ref["dg"], heads_axes)
    if gr.get("dS0") is not None:
        errs["dS0"] = slice_rel_err(gr["dS0"], ref["dS0"], (0, 1))
    bad = {n: e for n, e in errs.items() if not e <= tol}
    assert not bad, (bad, errs)


@pytest.mark.parametrize("variant", VARS)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 128), (128, 64), (64, 64)])
@pytest.mark.parametrize("T", [1, 63, 64, 65, 200])
def test_bwd_small(variant, dtype, dk, dv, T):
    announce("bwd_small", variant, dtype, dk, dv, T)
    w = Workload("t", variant, dtype, B=2, H=2, T=T, dk=dk, dv=dv, random_s0=True, seed=41 + T)
    x = make_forward_inputs(w)
    dO, dST = _upstream(w, 7 + T)
    gr = _run(variant, dtype, w, x, dO, dST)
    ref = oracle_bwd(variant, x["q"], x["k"], x["v"], x["beta"], x["wgate"], x["g"], x["S0"], dO, dST)
    _check(variant, dtype, gr, ref)


@pytest.mark.parametrize("variant", ["kda", "gdn2", "fg2"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_bwd_gate_floor(variant, dtype):
    """Channel log-decays of -10 are clamped to -85/16 on load: every gradient
    equals the oracle's reverse mode on the clamped gates, except dg, which is
    zero where the gate was clamped (the clamp passes no gradient) and the
    oracle's elsewhere."""
    announce("bwd_gate_floor", variant, dtype)
    w = Workload("t", variant, dtype, B=2, H=2, T=130, dk=128, dv=64, random_s0=True, seed=47)
    x = make_forward_inputs(w)
    x["g"] = floor_gates(x["g"].shape, dtype, 8)
    dO, dST = _upstream(w, 13)
    gr = _run(variant, dtype, w, x, dO, dST)
    clamped = x["g"] < LOG_DECAY_FLOOR
    gc = np.maximum(x["g"], LOG_DECAY_FLOOR)
    ref = oracle_bwd(variant, x["q"], x["k"], x["v"], x["beta"], x["wgate"], gc, x["S0"], dO, dST)
    for n in gr:
        if gr[n] is not None:
            assert np.isfinite(gr[n]).all(), n
    assert (gr["dg"][clamped] == 0).all()
    ref["dg"] = np.where(clamped, 0.0, ref["dg"])
    _check(variant, dtype, gr, ref)


@pytest.mark.parametrize("variant", VARS)
def test_bwd_no_state_gradient(variant):
    """dS_T = NULL (zero) and dS0 not requested; zero initial state."""
    announce("bwd_no_state_gradient", variant)
    w = Workload("t", variant, "f32", B=1, H=3, T=130, dk=128, dv=128, seed=43)
    x = make_forward_inputs(w)
    dO, _ = _upstream(w, 9)
    gr = ops.delta_bwd(variant, dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["beta"]), dev(dO),
                       g=dev(x["g"]), wgate=dev(x["wgate"]), want_dS0=False)
    torch.cuda.synchronize()
    assert gr["dS0"] is None
    gr = {n: host(t) for n, t in gr.items()}
    ref = oracle_bwd(variant, x["q"], x["k"], x["v"], x["beta"], x["wgate"], x["g"], None, dO, None)
    _check(variant, "f32", gr, ref)


@pytest.mark.parametrize("variant", ["gdn", "kda", "gdn2", "fg2"])
def test_bwd_long_all_heads(variant):
    """bf16, B=2, H=16, T=1024, d=128: every head checked against the oracle."""
    announce("bwd_long", variant)
    w = Workload("t", variant, "bf16", B=2, H=16, T=1024, dk=128, dv=128, random_s0=True, seed=44)
    x = make_forward_inputs(w)
    dO, dST = _upstream(w, 11)
    gr = _run(variant, "bf16", w, x, dO, dST)
    ref = bwd_all_heads(variant, {**x, "dO": dO, "dS_T": dST}, w.B, w.H)
    _check(variant, "bf16", gr, ref)


def test_bwd_headline_all_heads():
    """GDN, bf16, B=4, H=16, T=4096, d=128 with no initial state and no final-state
    gradient, as the backward is timed: every gradient of all 64 heads against the
    oracle."""
    w = WORKLOADS["gdn_bf16_b4_h16_t4096_d128"]
    announce("bwd_headline", w.name)
    x = make_forward_inputs(w)
    assert x["S0"] is None
    dO, _ = _upstream(w, 17)
    gr = _run("gdn", "bf16", w, x, dO, None)
    ref = bwd_all_heads("gdn", {**x, "dO": dO, "dS_T": None}, w.B, w.H)
    _check("gdn", "bf16", gr, ref)


def test_bwd_deterministic():
    w = Workload("t", "kda", "bf16", B=1, H=2, T=300, dk=128, dv=128, random_s0=True, seed=45)
    x = make_forward_inputs(w)
    dO, dST = _upstream(w, 12)
    a = _run("kda", "bf16", w, x, dO, dST)
    b = _run("kda", "bf16", w, x, dO, dST)
    for n in a:
        assert np.array_equal(a[n], b[n]), n


@pytest.mark.parametrize("variant", ["kda", "gdn2", "fg2"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_bwd_strong_channel_gates(variant, dtype):
    """Log-decays scaled by 3 (16-token sums near -35, single gates down to the
    -85/16 floor): the block-reference factors of the pairwise sums then reach
    e^{35} inside a block."""
    announce("bwd_strong_gates", variant, dtype)
    w = Workload("t", variant, dtype, B=1, H=2, T=200, dk=128, dv=128, random_s0=True, seed=46)
    x = make_forward_inputs(w, gate_scale=3.0)
    dO, dST = _upstream(w, 13)
    gr = _run(variant, dtype, w, x, dO, dST)
    ref = oracle_bwd(variant, x["q"], x["k"], x["v"], x["beta"], x["wgate"], x["g"], x["S0"], dO, dST)
    _check(variant, dtype, gr, ref)


@pytest.mark.parametrize("variant", VARS)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("H,Hk", [(4, 2), (4, 1)])
def test_bwd_grouped_heads(variant, dtype, H, Hk):
    """Grouped query/key heads: dq and dk summed over each group of value heads."""
    announce("bwd_grouped", variant, dtype, H, Hk)
    w = Workload("t", variant, dtype, B=2, H=H, T=130, dk=128, dv=64, random_s0=True, seed=47)
    x = make_forward_inputs(w, qk_heads=Hk)
    dO, dST = _upstream(w, 14)
    gr = _run(variant, dtype, w, x, dO, dST)
    assert gr["dq"].shape == (2, 130, Hk, 128)
    ref = oracle_bwd(variant, x["q"], x["k"], x["v"], x["beta"], x["wgate"], x["g"], x["S0"], dO, dST)
    _check(variant, dtype, gr, ref)


@pytest.mark.parametrize("variant", VARS)
def test_autograd_function(variant):
    """torch.autograd through delta_rule (forward and backward in the library's kernels)
    against the oracle's reverse mode, with grouped query/key heads."""
    from recurrent_memory_amd.autograd import delta_rule
    announce("autograd", variant)
    w = Workload("t", variant, "f32", B=1, H=4, T=100, dk=64, dv=64, random_s0=True, seed=48)
    x = make_forward_inputs(w, qk_heads=2)
    dO, dST = _upstream(w, 15)
    leaves = {n: (None if a is None else dev(a).requires_grad_(True))
              for n, a in x.items() if n != "S0"}
    S0 = dev(x["S0"]).requires_grad_(True)
    o, S = delta_rule(variant, leaves["q"], leaves["k"], leaves["v"], leaves["beta"], g=leaves["g"],
                      wgate=leaves["wgate"], S0=S0)
    (o * dev(dO)).sum().backward(retain_graph=True)
    (S * dev(dST)).sum().backward()
    ref = oracle_bwd(variant, x["q"], x["k"], x["v"], x["beta"], x["wgate"], x["g"], x["S0"], dO, dST)
    got = {"dq": leaves["q"].grad, "dk": leaves["k"].grad, "dv": leaves["v"].grad,
           "dbeta": leaves["beta"].grad, "dwgate": None if leaves["wgate"] is None else leaves["wgate"].grad,
           "dg": None if leaves["g"] is None else leaves["g"].grad, "dS0": S0.grad}
    _check(variant, "f32", {n: (None if t is None else host(t)) for n, t in got.items()}, ref)


@pytest.mark.parametrize("variant", VARS)
def test_bwd_many_heads(variant):
    """B*H = 330 heads: the chain kernels' XCD-aware head map with a partial last
    group of 8 and more workgroups than CUs; every head checked against the oracle."""
    announce("bwd_many_heads", variant)
    w = Workload("t", variant, "bf16", B=6, H=55, T=70, dk=64, dv=64, random_s0=True, seed=49)
    x = make_forward_inputs(w)
    dO, dST = _upstream(w, 16)
    gr = _run(variant, "bf16", w, x, dO, dST)
    ref = bwd_all_heads(variant, {**x, "dO": dO, "dS_T": dST}, w.B, w.H)
    _check(variant, "bf16", gr, ref)
