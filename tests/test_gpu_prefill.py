"""Chunkwise forward on the GPU against the token-by-token oracle."""
import dataclasses

import numpy as np
import pytest
import torch

from gpu_util import LOG_DECAY_FLOOR, TOL, announce, dev, errs, floor_gates, gpu_fwd, host, slice_rel_err
from oracle_pool import fwd_all_heads
from oracle import delta_fwd as oracle_fwd
from recurrent_memory_amd import ops
from recurrent_memory_amd.inputs import WORKLOADS, Workload, make_forward_inputs, round_to_bf16

pytestmark = pytest.mark.gpu

BUILT_VARIANTS = ["deltanet", "gdn", "kda", "gdn2", "fg2"]


def _check(variant, dtype, x, tol=None, **kw):
    o, S = gpu_fwd(variant, x, dtype, **kw)
    o_ref, S_ref = oracle_fwd(variant, **x)
    eo, es = errs(o, S, o_ref, S_ref)
    tol = TOL[dtype] if tol is None else tol
    assert eo <= tol and es <= tol, (eo, es)
    return eo, es


@pytest.mark.parametrize("variant", BUILT_VARIANTS)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128), (64, 128), (128, 64)])
@pytest.mark.parametrize("T", [1, 63, 64, 65, 200])
def test_small_shapes(variant, dtype, dk, dv, T):
    announce("prefill_small", variant, dtype, dk, dv, T)
    w = Workload("t", variant, dtype, B=2, H=3, T=T, dk=dk, dv=dv, random_s0=True, seed=T + dk)
    _check(variant, dtype, make_forward_inputs(w))


@pytest.mark.parametrize("variant", BUILT_VARIANTS)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_weak_decay_long_carry(variant, dtype):
    """Weak decay (g/16) so the state carries across many chunks."""
    announce("prefill_weak_decay", variant, dtype)
    w = Workload("t", variant, dtype, B=1, H=4, T=700, dk=128, dv=128, random_s0=True, seed=5)
    _check(variant, dtype, make_forward_inputs(w, gate_scale=1 / 16))


def test_deltanet_fp32_workload_full():
    w = WORKLOADS["deltanet_fp32_t256_d64"]
    announce("prefill_full", w.name)
    x = make_forward_inputs(w)
    eo, es = _check("deltanet", "f32", x)
    assert eo <= 1e-4


def test_gdn_bf16_workload_full_all_heads():
    """The headline workload at full size, every (batch, head) sequence checked
    against the oracle end to end (oracle heads in a process pool)."""
    w = WORKLOADS["gdn_bf16_b4_h16_t4096_d128"]
    announce("prefill_full", w.name)
    x = make_forward_inputs(w)
    o, S = gpu_fwd("gdn", x, "bf16")
    o_ref, S_ref = fwd_all_heads("gdn", x, w.B, w.H)
    eo, es = errs(o, S, o_ref, S_ref)
    assert eo <= TOL["bf16"] and es <= TOL["bf16"], (eo, es)


@pytest.mark.parametrize("name,variant", [("kda_bf16_b2_h16_t8192_d128", "kda"),
                                          ("gdn2_bf16_b1_h16_t32768_d128", "gdn2"),
                                          ("kda_bf16_b2_h16_t8192_d128", "fg2")])
def test_channel_decay_workloads_full_all_heads(name, variant):
    """KDA and Gated DeltaNet-2 workloads at full size (FG^2-GDN at the KDA shape),
    every (batch, head) sequence checked against the oracle end to end."""
    w = dataclasses.replace(WORKLOADS[name], variant=variant)
    announce("prefill_full", w.name, variant)
    x = make_forward_inputs(w)
    o, S = gpu_fwd(variant, x, "bf16")
    o_ref, S_ref = fwd_all_heads(variant, x, w.B, w.H)
    eo, es = errs(o, S, o_ref, S_ref)
    assert eo <= TOL["bf16"] and es <= TOL["bf16"], (eo, es)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gdn2_reduces_to_kda_on_gpu(dtype):
    """Gated DeltaNet-2 with erase and write gates equal to beta reproduces KDA."""
    announce("gdn2_reduction", dtype)
    w = Workload("t", "kda", dtype, B=2, H=3, T=300, dk=128, dv=128, random_s0=True, seed=12)
    x = make_forward_inputs(w, gate_scale=1 / 4)
    o_kda, S_kda = gpu_fwd("kda", x, dtype)
    b = np.repeat(x["beta"][..., None], 128, axis=-1)
    x2 = {**x, "beta": b, "wgate": b.copy()}
    o2, S2 = gpu_fwd("gdn2", x2, dtype)
    tol = 1e-5 if dtype == "f32" else 2e-2
    assert slice_rel_err(o2, o_kda, (0, 2)) <= tol
    assert slice_rel_err(S2, S_kda, (0, 1)) <= tol


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_fg2_reduces_to_kda_on_gpu(dtype):
    """FG^2-GDN with the step size beta repeated over the key channels reproduces KDA."""
    announce("fg2_reduction", dtype)
    w = Workload("t", "kda", dtype, B=2, H=3, T=300, dk=128, dv=128, random_s0=True, seed=14)
    x = make_forward_inputs(w, gate_scale=1 / 4)
    o_kda, S_kda = gpu_fwd("kda", x, dtype)
    x2 = {**x, "beta": np.repeat(x["beta"][..., None], 128, axis=-1)}
    o2, S2 = gpu_fwd("fg2", x2, dtype)
    tol = 1e-5 if dtype == "f32" else 2e-2
    assert slice_rel_err(o2, o_kda, (0, 2)) <= tol
    assert slice_rel_err(S2, S_kda, (0, 1)) <= tol


@pytest.mark.parametrize("variant", ["kda", "gdn2", "fg2"])
def test_channel_decay_strong_gates(variant):
    """Per-channel log-decays down to -4 per token (decay e^-4, so up to -64 summed
    over a 16-token block): the split exponentials stay inside the fp32 range
    because each is taken relative to a block boundary."""
    announce("strong_gates", variant)
    for dtype in ("f32", "bf16"):
        w = Workload("t", variant, dtype, B=1, H=2, T=150, dk=64, dv=64, random_s0=True, seed=13)
        x = make_forward_inputs(w)
        rng = np.random.default_rng(5)
        g = (-rng.uniform(0, 4, x["g"].shape)).astype(np.float32)
        x["g"] = g if dtype == "f32" else round_to_bf16(g)
        _check(variant, dtype, x)


@pytest.mark.parametrize("variant", ["kda", "gdn2", "fg2"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk", [64, 128])
def test_channel_decay_gate_floor(variant, dtype, dk):
    """Per-token log-decays of -10 (16 tokens would sum to -160, past the range of
    the block-relative split exponentials): every gate is clamped to -85/16 when
    it is loaded, so the outputs are finite and equal the oracle's on the clamped
    gates (in fp32 measurably closer to those than to the oracle's on the raw
    gates)."""
    announce("gate_floor", variant, dtype, dk)
    w = Workload("t", variant, dtype, B=1, H=2, T=150, dk=dk, dv=dk, random_s0=True, seed=17)
    x = make_forward_inputs(w)
    x["g"] = floor_gates(x["g"].shape, dtype, 6)
    o, S = gpu_fwd(variant, x, dtype)
    assert np.isfinite(o).all() and np.isfinite(S).all()
    xc = dict(x, g=np.maximum(x["g"], LOG_DECAY_FLOOR))
    o_ref, S_ref = oracle_fwd(variant, **xc)
    eo, es = errs(o, S, o_ref, S_ref)
    assert eo <= TOL[dtype] and es <= TOL[dtype], (eo, es)
    if dtype == "f32":   # the clamp is in effect: fp32 separates the two references
        o_raw, S_raw = oracle_fwd(variant, **x)
        assert max(errs(o, S, o_raw, S_raw)) > 10 * max(eo, es)


def test_unit_write_full_size_no_oracle():
    """beta = 1, q = k, unit keys: o_t = v_t exactly in exact arithmetic, at full size.
    In bf16 the rounded key is not exactly unit-norm, which bounds the error."""
    w = WORKLOADS["gdn_bf16_b4_h16_t4096_d128"]
    announce("prefill_unit_write", w.name)
    x = make_forward_inputs(w)
    x["beta"] = np.ones_like(x["beta"])
    x["q"] = x["k"]
    o, _ = gpu_fwd("gdn", x, "bf16", want_state=False)
    knorm2 = (x["k"].astype(np.float64) ** 2).sum(-1)
    assert np.abs(knorm2 - 1).max() < 8e-3
    assert slice_rel_err(o, x["v"], (0, 2)) <= 2e-2


def test_in_place_state_and_split_sequence():
    """S_T written over S0, and running [0, T1) then [T1, T) equals [0, T)."""
    announce("prefill_in_place_split")
    w = Workload("t", "gdn", "f32", B=2, H=2, T=300, dk=128, dv=128, random_s0=True, seed=9)
    x = make_forward_inputs(w, gate_scale=1 / 8)
    o_full, S_full = gpu_fwd("gdn", x, "f32")
    per_tok = ("q", "k", "v", "beta", "g")
    xa = {n: x[n][:, :130] for n in per_tok}
    xa["S0"], xa["wgate"] = x["S0"], None
    S0 = dev(x["S0"], "f32")
    o_a, _ = ops.delta_fwd("gdn", *(dev(xa[n], "f32") for n in ("q", "k", "v", "beta")),
                           g=dev(xa["g"], "f32"), S0=S0, S_T=S0)
    o_b, _ = ops.delta_fwd("gdn", *(dev(x[n][:, 130:], "f32") for n in ("q", "k", "v", "beta")),
                           g=dev(x["g"][:, 130:], "f32"), S0=S0, S_T=S0)
    torch.cuda.synchronize()
    o_split = np.concatenate([host(o_a), host(o_b)], axis=1)
    assert slice_rel_err(o_split, o_full, (0, 2)) <= 1e-5
    assert slice_rel_err(host(S0), S_full, (0, 1)) <= 1e-5


def test_deterministic():
    announce("prefill_deterministic")
    w = Workload("t", "gdn", "bf16", B=2, H=4, T=333, dk=128, dv=128, random_s0=True, seed=3)
    x = make_forward_inputs(w)
    o1, S1 = gpu_fwd("gdn", x, "bf16")
    o2, S2 = gpu_fwd("gdn", x, "bf16")
    assert np.array_equal(o1, o2) and np.array_equal(S1, S2)


def test_decode_continues_prefill():
    """Decode of token T+1 from the prefill state equals prefill over T+1 tokens."""
    announce("decode_after_prefill")
    w = Workload("t", "gdn", "f32", B=2, H=3, T=129, dk=128, dv=128, random_s0=True, seed=4)
    x = make_forward_inputs(w)
    o_full, S_full = gpu_fwd("gdn", x, "f32")
    xa = {n: (None if x[n] is None else x[n][:, :128]) for n in ("q", "k", "v", "beta", "wgate", "g")}
    xa["S0"] = x["S0"]
    _, S_a = gpu_fwd("gdn", xa, "f32")
    S = dev(S_a.astype(np.float32), "f32")
    step = {n: dev(x[n][:, 128], "f32") for n in ("q", "k", "v", "beta", "g")}
    o = ops.delta_decode("gdn", step["q"], step["k"], step["v"], step["beta"], S, g=step["g"])
    torch.cuda.synchronize()
    assert slice_rel_err(host(o), o_full[:, 128], (0, 1)) <= 1e-5
    assert slice_rel_err(host(S), S_full, (0, 1)) <= 1e-5


def _per_token(x, lo, hi):
    return {n: (None if x.get(n) is None else x[n][:, lo:hi]) for n in ("q", "k", "v", "beta", "wgate", "g")}


@pytest.mark.parametrize("variant", BUILT_VARIANTS)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_split_sequence_in_place_all_forms(variant, dtype):
    """Chunked prefill from a cached state: [0, 100) then [100, 261) with the
    state updated in place (S_T = S0) matches the oracle over [0, 261).  The
    split falls inside a chunk of both calls."""
    announce("prefill_split_in_place", variant, dtype)
    w = Workload("t", variant, dtype, B=2, H=3, T=261, dk=128, dv=64, random_s0=True, seed=21)
    x = make_forward_inputs(w, gate_scale=1 / 4)
    o_ref, S_ref = oracle_fwd(variant, **x)
    S = dev(x["S0"], "f32")
    outs = []
    for lo, hi in ((0, 100), (100, 261)):
        part = _per_token(x, lo, hi)
        o, _ = ops.delta_fwd(variant, *(dev(part[n], dtype) for n in ("q", "k", "v", "beta")),
                             wgate=dev(part["wgate"], dtype), g=dev(part["g"], dtype), S0=S, S_T=S)
        outs.append(o)
    torch.cuda.synchronize()
    o_split = np.concatenate([host(t) for t in outs], axis=1)
    eo, es = errs(o_split, host(S), o_ref, S_ref)
    assert eo <= TOL[dtype] and es <= TOL[dtype], (eo, es)


@pytest.mark.parametrize("variant", BUILT_VARIANTS)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_continues_prefill_all_forms(variant, dtype):
    """Prefill of 97 tokens hands its state to three decode steps; the four
    outputs of the decode steps and the final state match the oracle over 100
    tokens."""
    announce("decode_after_prefill_all", variant, dtype)
    w = Workload("t", variant, dtype, B=2, H=2, T=100, dk=64, dv=128, random_s0=True, seed=22)
    x = make_forward_inputs(w, gate_scale=1 / 2)
    o_ref, S_ref = oracle_fwd(variant, **x)
    pre = _per_token(x, 0, 97)
    S = dev(x["S0"], "f32")
    ops.delta_fwd(variant, *(dev(pre[n], dtype) for n in ("q", "k", "v", "beta")),
                  wgate=dev(pre["wgate"], dtype), g=dev(pre["g"], dtype), S0=S, S_T=S)
    outs = []
    for t in range(97, 100):
        step = {n: (None if x.get(n) is None else x[n][:, t]) for n in ("q", "k", "v", "beta", "wgate", "g")}
        o = ops.delta_decode(variant, *(dev(step[n], dtype) for n in ("q", "k", "v", "beta")), S,
                             wgate=dev(step["wgate"], dtype), g=dev(step["g"], dtype))
        outs.append(host(o))
    torch.cuda.synchronize()
    o_dec = np.stack(outs, axis=1)
    eo, es = errs(o_dec, host(S), o_ref[:, 97:], S_ref)
    assert eo <= TOL[dtype] and es <= TOL[dtype], (eo, es)


@pytest.mark.parametrize("variant", BUILT_VARIANTS)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_many_heads_several_dispatch_rounds(variant, dtype):
    """B*H = 330 heads (not a multiple of 8), so every kernel's grid holds more
    workgroups than there are CUs and the XCD-aware head map has a partial last
    group; every head checked against the oracle."""
    announce("prefill_many_heads", variant, dtype)
    w = Workload("t", variant, dtype, B=6, H=55, T=70, dk=64, dv=64, random_s0=True, seed=31)
    x = make_forward_inputs(w)
    o, S = gpu_fwd(variant, x, dtype)
    o_ref, S_ref = fwd_all_heads(variant, x, w.B, w.H)
    eo, es = errs(o, S, o_ref, S_ref)
    assert eo <= TOL[dtype] and es <= TOL[dtype], (eo, es)
