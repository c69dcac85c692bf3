"""The chunkwise backward model (chunkref_bwd.py) against the oracle's token-level
reverse mode: every gradient, for chunk lengths 1, 16, 37 and 64, ragged tails,
DeltaNet, GDN and KDA."""
import numpy as np
import pytest

from chunkref_bwd import chunk_backward, chunk_forward
from oracle import delta_bwd, delta_fwd


def _one_head(rng, variant, T, dk, dv):
    q = rng.standard_normal((1, T, 1, dk)) / np.sqrt(dk)
    k = rng.standard_normal((1, T, 1, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((1, T, 1, dv))
    beta = rng.uniform(0, 1, (1, T, 1))
    g = {"deltanet": None, "gdn": -rng.uniform(0, 0.5, (1, T, 1)),
         "kda": -rng.uniform(0, 0.5, (1, T, 1, dk))}[variant]
    S0 = rng.standard_normal((1, 1, dv, dk)) * 0.3
    dO = rng.standard_normal((1, T, 1, dv))
    dST = rng.standard_normal((1, 1, dv, dk))
    return dict(q=q, k=k, v=v, beta=beta, g=g, S0=S0), dO, dST


def _gfull(variant, g, T, dk):
    if g is None:
        return np.zeros((T, dk))
    if variant == "gdn":
        return np.repeat(g[0, :, 0, None], dk, axis=1)
    return g[0, :, 0]


@pytest.mark.parametrize("variant", ["deltanet", "gdn", "kda"])
@pytest.mark.parametrize("C,T", [(1, 9), (16, 50), (37, 80), (64, 150), (64, 64)])
def test_chunk_backward_matches_oracle(variant, C, T):
    rng = np.random.default_rng(C * 1000 + T)
    dk, dv = 6, 5
    x, dO, dST = _one_head(rng, variant, T, dk, dv)
    gf = _gfull(variant, x["g"], T, dk)
    o, S, _ = chunk_forward(x["q"][0, :, 0], x["k"][0, :, 0], x["v"][0, :, 0], x["beta"][0, :, 0],
                            gf, x["S0"][0, 0], C)
    o_ref, S_ref = delta_fwd(variant, **x)
    np.testing.assert_allclose(o, o_ref[0, :, 0], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(S, S_ref[0, 0], rtol=1e-10, atol=1e-12)
    dq, dk_, dv_, db, dg, dS0 = chunk_backward(
        x["q"][0, :, 0], x["k"][0, :, 0], x["v"][0, :, 0], x["beta"][0, :, 0], gf, x["S0"][0, 0],
        dO[0, :, 0], dST[0, 0], C)
    ref = delta_bwd(variant, **x, dO=dO, dS_T=dST)
    tol = dict(rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(dq, ref["dq"][0, :, 0], **tol)
    np.testing.assert_allclose(dk_, ref["dk"][0, :, 0], **tol)
    np.testing.assert_allclose(dv_, ref["dv"][0, :, 0], **tol)
    np.testing.assert_allclose(db, ref["dbeta"][0, :, 0], **tol)
    np.testing.assert_allclose(dS0, ref["dS0"][0, 0], **tol)
    if variant == "gdn":
        np.testing.assert_allclose(dg.sum(axis=1), ref["dg"][0, :, 0], **tol)
    elif variant == "kda":
        np.testing.assert_allclose(dg, ref["dg"][0, :, 0], **tol)


@pytest.mark.parametrize("C,T", [(1, 7), (16, 40), (37, 80), (64, 150)])
def test_split_gate_chunk_backward_matches_oracle(C, T):
    from chunkref_bwd import chunk_backward2, chunk_forward2
    rng = np.random.default_rng(C * 77 + T)
    dk, dv = 6, 5
    q = rng.standard_normal((1, T, 1, dk)) / np.sqrt(dk)
    k = rng.standard_normal((1, T, 1, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((1, T, 1, dv))
    b = rng.uniform(0, 1, (1, T, 1, dk))
    w = rng.uniform(0, 1, (1, T, 1, dv))
    g = -rng.uniform(0, 0.5, (1, T, 1, dk))
    S0 = rng.standard_normal((1, 1, dv, dk)) * 0.3
    dO = rng.standard_normal((1, T, 1, dv))
    dST = rng.standard_normal((1, 1, dv, dk))
    x = dict(q=q, k=k, v=v, beta=b, wgate=w, g=g, S0=S0)
    h = lambda a: a[0, :, 0]  # noqa: E731
    o, S, _ = chunk_forward2(h(q), h(k), h(v), h(b), h(w), h(g), S0[0, 0], C)
    o_ref, S_ref = delta_fwd("gdn2", **x)
    np.testing.assert_allclose(o, o_ref[0, :, 0], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(S, S_ref[0, 0], rtol=1e-10, atol=1e-12)
    got = chunk_backward2(h(q), h(k), h(v), h(b), h(w), h(g), S0[0, 0], h(dO), dST[0, 0], C)
    ref = delta_bwd("gdn2", **x, dO=dO, dS_T=dST)
    tol = dict(rtol=1e-9, atol=1e-11)
    for mine, theirs in (("dq", "dq"), ("dk", "dk"), ("dv", "dv"), ("db", "dbeta"),
                         ("dw", "dwgate"), ("dg", "dg")):
        np.testing.assert_allclose(got[mine], h(ref[theirs]), err_msg=mine, **tol)
    np.testing.assert_allclose(got["dS0"], ref["dS0"][0, 0], **tol)
