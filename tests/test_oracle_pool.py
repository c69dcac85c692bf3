"""The per-head process pool used by the full-size GPU tests reassembles exactly
what the oracle computes over all heads at once."""
import numpy as np

from oracle import delta_bwd, delta_fwd, ttt_pre_fwd
from oracle_pool import bwd_all_heads, fwd_all_heads, ttt_all_heads
from recurrent_memory_amd.inputs import Workload, make_forward_inputs, make_ttt_inputs


def test_forward_grouped_heads_match_whole_call():
    w = Workload("t", "kda", "f32", B=2, H=4, T=37, dk=16, dv=8, random_s0=True, seed=3)
    x = make_forward_inputs(w, qk_heads=2)
    o, S = fwd_all_heads("kda", x, w.B, w.H)
    o_ref, S_ref = delta_fwd("kda", **x)
    assert np.array_equal(o, o_ref) and np.array_equal(S, S_ref)


def test_backward_matches_whole_call():
    w = Workload("t", "gdn2", "f32", B=2, H=3, T=20, dk=8, dv=8, random_s0=True, seed=4)
    x = make_forward_inputs(w)
    rng = np.random.default_rng(5)
    dO = rng.standard_normal((w.B, w.T, w.H, w.dv))
    dST = rng.standard_normal((w.B, w.H, w.dv, w.dk))
    got = bwd_all_heads("gdn2", {**x, "dO": dO, "dS_T": dST}, w.B, w.H)
    ref = delta_bwd("gdn2", x["q"], x["k"], x["v"], x["beta"], x["wgate"], x["g"], x["S0"], dO, dST)
    for n, a in ref.items():
        assert (a is None and got[n] is None) or np.allclose(got[n], a, rtol=0, atol=1e-12), n


def test_ttt_matches_whole_call():
    w = Workload("t", "gdn", "f32", B=1, H=3, T=25, dk=8, dv=8, seed=6)
    x = make_ttt_inputs(w)
    got = ttt_all_heads("gdn", x, w.B, w.H)
    ref = ttt_pre_fwd("gdn", x["q"], x["k"], x["v"], x["beta1"], x["g1"], x["beta2"], x["g2"], x["A0"], x["B0"])
    for a, r in zip(got, ref):
        assert np.allclose(a, r, rtol=0, atol=1e-12)
