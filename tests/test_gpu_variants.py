"""Grouped value heads and exact-flow (EFLA) step sizes on the GPU against the oracle.

Grouped value heads: q and k carry H_k heads, v, the gates and the state H; value
head h reads query/key head h // (H / H_k).  Every forward kernel (fp32 and bf16,
scalar and channel-wise decay) and the decode kernel are run with H_k < H.

EFLA: delta_efla_beta turns (k, beta) into the exact-flow step sizes; the tests
check them element by element and then run the forward and decode paths on them.
"""
import numpy as np
import pytest
import torch

from oracle_pool import fwd_all_heads
from gpu_util import TOL, announce, dev, errs, gpu_fwd, host, slice_rel_err
from oracle import delta_decode as oracle_decode
from oracle import delta_fwd as oracle_fwd
from oracle import efla_step_size
from recurrent_memory_amd import ops
from recurrent_memory_amd.inputs import WORKLOADS, Workload, make_decode_inputs, make_forward_inputs

pytestmark = pytest.mark.gpu

ALL = ["deltanet", "gdn", "kda", "gdn2", "fg2"]


def _oracle(variant, x, heads=None):
    """Oracle forward on all (batch, value head) pairs, or on ``heads`` = (b list, h list)."""
    if heads is None:
        return oracle_fwd(variant, x["q"], x["k"], x["v"], x["beta"], x["wgate"], x["g"], x["S0"])
    bs, hs = heads
    H, Hk = x["v"].shape[2], x["q"].shape[2]
    G = H // Hk
    sel = lambda a, h: None if a is None else a[bs][:, :, [h]]  # noqa: E731
    outs, states = [], []
    for h in hs:
        qk = lambda a: a[bs][:, :, [h // G]]  # noqa: E731
        S0 = None if x["S0"] is None else x["S0"][bs][:, [h]]
        o, S = oracle_fwd(variant, qk(x["q"]), qk(x["k"]), sel(x["v"], h), sel(x["beta"], h),
                          sel(x["wgate"], h), sel(x["g"], h), S0)
        outs.append(o)
        states.append(S)
    return np.concatenate(outs, axis=2), np.concatenate(states, axis=1)


@pytest.mark.parametrize("variant", ALL)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("H,Hk,T,d", [(4, 2, 200, 128), (4, 1, 64, 128), (6, 3, 131, 64)])
def test_grouped_forward(variant, dtype, H, Hk, T, d):
    announce("grouped_forward", variant, dtype, H, Hk, T, d)
    w = Workload("t", variant, dtype, B=2, H=H, T=T, dk=d, dv=d, random_s0=True, seed=31)
    x = make_forward_inputs(w, qk_heads=Hk)
    assert x["q"].shape[2] == Hk and x["v"].shape[2] == H
    o, S = gpu_fwd(variant, x, dtype)
    o_ref, S_ref = _oracle(variant, x)
    eo, es = errs(o, S, o_ref, S_ref)
    assert eo <= TOL[dtype] and es <= TOL[dtype], (eo, es)


def test_grouped_forward_full_size_all_heads():
    """GDN bf16 at B=4, H=16, T=4096, d=128 with 8 query/key heads (pairs of value
    heads), the launch the headline forward uses; every value head checked."""
    w = Workload("t", "gdn", "bf16", B=4, H=16, T=4096, dk=128, dv=128, seed=32)
    announce("grouped_forward_full", w)
    x = make_forward_inputs(w, qk_heads=8)
    o, S = gpu_fwd("gdn", x, "bf16")
    o_ref, S_ref = fwd_all_heads("gdn", x, w.B, w.H)
    eo, es = errs(o, S, o_ref, S_ref)
    assert eo <= TOL["bf16"] and es <= TOL["bf16"], (eo, es)


@pytest.mark.parametrize("variant", ALL)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("H,Hk", [(4, 2), (4, 1)])
def test_grouped_decode(variant, dtype, H, Hk):
    announce("grouped_decode", variant, dtype, H, Hk)
    w = Workload("t", variant, dtype, B=3, H=H, T=1, dk=128, dv=128, random_s0=True, seed=33)
    d = make_decode_inputs(w, 3, qk_heads=Hk)
    S = dev(d["S"], "f32")
    S_ref = d["S"].astype(np.float64)
    for s in d["steps"]:
        t = {n: dev(a, dtype) for n, a in s.items()}
        o = ops.delta_decode(variant, t["q"], t["k"], t["v"], t["beta"], S, wgate=t["wgate"], g=t["g"])
        torch.cuda.synchronize()
        o_ref, S_ref = oracle_decode(variant, **s, S=S_ref)
        assert slice_rel_err(host(o), o_ref, (0, 1)) <= TOL[dtype]
    assert slice_rel_err(host(S), S_ref, (0, 1)) <= 1e-5


# ------------------------------------------------------------------ EFLA


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("Hk", [4, 2, 1])
@pytest.mark.parametrize("key_norm", [1.0, 2.5, 0.05])
def test_efla_step_sizes(dtype, d, Hk, key_norm):
    announce("efla_step_sizes", dtype, d, Hk, key_norm)
    w = Workload("t", "gdn", dtype, B=2, H=4, T=300, dk=d, dv=d, seed=34)
    x = make_forward_inputs(w, qk_heads=Hk, key_norm=key_norm)
    k, beta = dev(x["k"], dtype), dev(x["beta"], dtype)
    c = host(ops.efla_beta("gdn", k, beta))
    ref = efla_step_size(x["k"], x["beta"])
    rel = np.abs(c - ref) / np.abs(ref)
    # fp32: ||k||^2 summed in fp32 and expm1f; bf16: one rounding of the fp32 value
    assert rel.max() <= (2e-6 if dtype == "f32" else 2.0 ** -8), rel.max()
    # in place, and the decode layout (T = 1) on one token
    ops.efla_beta("gdn", k, beta, out=beta)
    torch.cuda.synchronize()
    assert np.array_equal(host(beta), c)
    c1 = host(ops.efla_beta("gdn", k[:, 7].contiguous(), dev(x["beta"][:, 7], dtype)))
    assert np.array_equal(c1, c[:, 7])


def test_efla_step_sizes_full_size():
    """The timed EFLA workload (bf16, B=4, H=16, T=4096, d=128): every step size
    against the oracle's."""
    w = WORKLOADS["gdn_bf16_b4_h16_t4096_d128"]
    announce("efla_full", w.name)
    x = make_forward_inputs(w)
    c = host(ops.efla_beta("gdn", dev(x["k"], "bf16"), dev(x["beta"], "bf16")))
    ref = efla_step_size(x["k"], x["beta"])
    assert c.shape == ref.shape
    assert (np.abs(c - ref) / np.abs(ref)).max() <= 2.0 ** -8


def test_efla_zero_keys_keep_beta():
    """A zero key has no flow direction: the step size stays beta exactly."""
    k = torch.zeros((1, 5, 2, 128), dtype=torch.float32, device="cuda")
    beta = torch.rand((1, 5, 2), dtype=torch.float32, device="cuda")
    assert torch.equal(ops.efla_beta("deltanet", k, beta), beta)


@pytest.mark.parametrize("variant", ["deltanet", "gdn", "kda"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_efla_forward(variant, dtype):
    """delta_efla_beta then delta_fwd against the oracle run with exact-flow step sizes,
    high-energy keys (norm 2), 2 query/key heads over 4 value heads."""
    announce("efla_forward", variant, dtype)
    w = Workload("t", variant, dtype, B=2, H=4, T=257, dk=128, dv=128, random_s0=True, seed=35)
    x = make_forward_inputs(w, qk_heads=2, key_norm=2.0)
    beta_eff = ops.efla_beta(variant, dev(x["k"], dtype), dev(x["beta"], dtype))
    o, S = ops.delta_fwd(variant, dev(x["q"], dtype), dev(x["k"], dtype), dev(x["v"], dtype),
                         beta_eff, g=dev(x["g"], dtype), S0=dev(x["S0"], "f32"))
    torch.cuda.synchronize()
    o_ref, S_ref = oracle_fwd(variant, x["q"], x["k"], x["v"], efla_step_size(x["k"], x["beta"]),
                              None, x["g"], x["S0"])
    eo, es = errs(host(o), host(S), o_ref, S_ref)
    assert eo <= TOL[dtype] and es <= TOL[dtype], (eo, es)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_efla_decode(dtype):
    announce("efla_decode", dtype)
    w = Workload("t", "gdn", dtype, B=8, H=4, T=1, dk=128, dv=128, random_s0=True, seed=36)
    d = make_decode_inputs(w, 2, key_norm=1.5)
    S = dev(d["S"], "f32")
    S_ref = d["S"].astype(np.float64)
    for s in d["steps"]:
        t = {n: dev(a, dtype) for n, a in s.items()}
        be = ops.efla_beta("gdn", t["k"], t["beta"])
        o = ops.delta_decode("gdn", t["q"], t["k"], t["v"], be, S, g=t["g"])
        torch.cuda.synchronize()
        o_ref, S_ref = oracle_decode("gdn", s["q"], s["k"], s["v"],
                                     efla_step_size(s["k"], s["beta"]), None, s["g"], S=S_ref)
        assert slice_rel_err(host(o), o_ref, (0, 1)) <= TOL[dtype]
    # the step sizes reach the kernel rounded to the input dtype (2^-9 relative for
    # bf16), the oracle's are exact: the state differs by that much of one write
    assert slice_rel_err(host(S), S_ref, (0, 1)) <= (2e-5 if dtype == "f32" else 4e-3)
