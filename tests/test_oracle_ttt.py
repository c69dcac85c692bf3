"""Pins of the oracle's DeltaTTT-pre (ttt_pre_fwd) against the delta-rule oracle and
the structure the DeltaTTT summary states.

- The second layer with no writes and B0 = I passes the query representation
  through: o_t = unit(silu(A_t q_t)), with A_t from the delta-rule oracle.
- Pre schedule (DeltaTTT summary, §4.1): the second layer's write key of token t
  is formed from the first layer's state before token t's write: it equals
  unit(silu(A_{t-1} D_t k_t)) with A_{t-1} the delta-rule oracle's state after
  t - 1 tokens.
- Two scans (Appendix A, chunkwise scan): the token-interleaved definition
  equals a first scan over A followed by an ordinary delta-rule scan over B with
  the formed keys and queries.
"""
import numpy as np
import pytest

from oracle import delta_fwd, ttt_pre_fwd


def _inputs(rng, variant, B=2, T=9, H=2, dk=5, dv=4):
    unit = lambda x: x / np.linalg.norm(x, axis=-1, keepdims=True)  # noqa: E731
    x = dict(q=unit(rng.standard_normal((B, T, H, dk))), k=unit(rng.standard_normal((B, T, H, dk))),
             v=rng.standard_normal((B, T, H, dv)), beta1=rng.uniform(0, 1, (B, T, H)),
             beta2=rng.uniform(0, 1, (B, T, H)),
             A0=0.3 * rng.standard_normal((B, H, dv, dk)), B0=0.3 * rng.standard_normal((B, H, dv, dv)))
    if variant == "gdn":
        x["g1"] = -rng.uniform(0, 1, (B, T, H))
        x["g2"] = -rng.uniform(0, 1, (B, T, H))
    return x


def _silu_unit(x):
    s = x / (1 + np.exp(-x))
    return s / np.linalg.norm(s, axis=-1, keepdims=True)


@pytest.mark.parametrize("variant", ["deltanet", "gdn"])
def test_identity_second_layer_passes_the_query_representation(variant):
    rng = np.random.default_rng(1)
    x = _inputs(rng, variant)
    x["beta2"] = np.zeros_like(x["beta2"])
    if variant == "gdn":
        x["g2"] = np.zeros_like(x["g2"])
    x["B0"] = np.broadcast_to(np.eye(4), x["B0"].shape).copy()
    o, A_T, _ = ttt_pre_fwd(variant, **x)
    o1, S1 = delta_fwd(variant, x["q"], x["k"], x["v"], x["beta1"], g=x.get("g1"), S0=x["A0"])
    np.testing.assert_allclose(o, _silu_unit(o1), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(A_T, S1, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("variant", ["deltanet", "gdn"])
def test_pre_schedule_write_key_uses_the_previous_state(variant):
    rng = np.random.default_rng(2)
    x = _inputs(rng, variant)
    _, _, _, h, z = ttt_pre_fwd(variant, **x, internals=True)
    o1, _ = delta_fwd(variant, x["q"], x["k"], x["v"], x["beta1"], g=x.get("g1"), S0=x["A0"])
    np.testing.assert_allclose(z, _silu_unit(o1), rtol=1e-12, atol=1e-13)   # read after the write
    for t in (0, 1, 5, 8):
        if t == 0:
            A_prev = x["A0"]
        else:
            cut = lambda a: None if a is None else a[:, :t]  # noqa: E731
            _, A_prev = delta_fwd(variant, cut(x["q"]), cut(x["k"]), cut(x["v"]), cut(x["beta1"]),
                                  g=cut(x.get("g1")), S0=x["A0"])
        a = np.exp(x["g1"][:, t]) if variant == "gdn" else np.ones(x["beta1"].shape[::2])
        r = np.einsum("bhvk,bhk->bhv", A_prev, x["k"][:, t]) * a[..., None]
        np.testing.assert_allclose(h[:, t], _silu_unit(r), rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("variant", ["deltanet", "gdn"])
def test_two_scans_equal_the_interleaved_definition(variant):
    rng = np.random.default_rng(3)
    x = _inputs(rng, variant, T=13)
    o, _, B_T, h, z = ttt_pre_fwd(variant, **x, internals=True)
    o2, S2 = delta_fwd(variant, z, h, x["v"], x["beta2"], g=x.get("g2"), S0=x["B0"])
    np.testing.assert_allclose(o, o2, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(B_T, S2, rtol=1e-12, atol=1e-13)


def test_changing_the_current_value_leaves_the_current_write_key():
    """Pre: the write key of token t does not see token t's first-layer write."""
    rng = np.random.default_rng(4)
    x = _inputs(rng, "gdn")
    _, _, _, h, _ = ttt_pre_fwd("gdn", **x, internals=True)
    x2 = {n: (a.copy() if isinstance(a, np.ndarray) else a) for n, a in x.items()}
    x2["v"][:, 4] += 3.0
    _, _, _, h2, _ = ttt_pre_fwd("gdn", **x2, internals=True)
    np.testing.assert_array_equal(h2[:, :5], h[:, :5])
    assert np.abs(h2[:, 5] - h[:, 5]).max() > 1e-3


# ---- the nonlinearity and the normalisation, pinned by values the mathematics fixes

def test_silu_values_fixed_by_the_definition():
    """silu(x) = x * sigmoid(x): silu(0) = 0, silu(ln 3) = (3/4) ln 3 (sigmoid(ln 3) =
    3/4), silu(-ln 3) = -(1/4) ln 3, silu(x) - silu(-x) = x, silu(x) -> x for large x
    and -> 0 for large -x."""
    from oracle.delta_oracle import _silu
    l3 = np.log(3.0)
    got = _silu(np.array([0.0, l3, -l3, 40.0, -40.0]))
    np.testing.assert_allclose(got[:3], [0.0, 0.75 * l3, -0.25 * l3], rtol=1e-15, atol=0)
    assert abs(got[3] - 40.0) < 1e-15 * 40 + 40 * np.exp(-40) and abs(got[4]) < 41 * np.exp(-40)
    x = np.linspace(-6, 6, 25)
    np.testing.assert_allclose(_silu(x) - _silu(-x), x, rtol=0, atol=1e-14)


def test_unit_rows_values_fixed_by_the_definition():
    """unit(x) = x / ||x||: (3, 4) -> (0.6, 0.8), norm 1, positive scaling leaves it,
    a zero row stays zero (no division by zero)."""
    from oracle.delta_oracle import _unit_rows
    got = _unit_rows(np.array([[3.0, 4.0], [0.0, 0.0], [-5.0, 0.0]]))
    np.testing.assert_allclose(got, [[0.6, 0.8], [0.0, 0.0], [-1.0, 0.0]], rtol=1e-15, atol=0)
    rng = np.random.default_rng(5)
    x = rng.standard_normal((7, 9))
    np.testing.assert_allclose(np.linalg.norm(_unit_rows(x), axis=-1), 1.0, rtol=1e-14)
    np.testing.assert_allclose(_unit_rows(2.5 * x), _unit_rows(x), rtol=1e-14)


def test_ttt_keys_and_queries_on_a_worked_example():
    """One token, d = 2, first layer A0 = [[ln 3, 0], [-ln 3, 0]], k = q = e_0, no
    first-layer write (beta1 = 0): the pre-write read is r = (ln 3, -ln 3), so the
    second layer's key and query are unit((3/4 ln 3, -1/4 ln 3)) = (3, -1)/sqrt(10);
    with B0 = 0 and beta2 = 1 the second layer stores v h^T and reads back v (h.z = 1)."""
    l3 = np.log(3.0)
    x = dict(q=np.array([1.0, 0.0]).reshape(1, 1, 1, 2), k=np.array([1.0, 0.0]).reshape(1, 1, 1, 2),
             v=np.array([0.7, -1.3]).reshape(1, 1, 1, 2), beta1=np.zeros((1, 1, 1)),
             beta2=np.ones((1, 1, 1)), A0=np.array([[l3, 0.0], [-l3, 0.0]]).reshape(1, 1, 2, 2),
             B0=np.zeros((1, 1, 2, 2)))
    o, A_T, B_T, h, z = ttt_pre_fwd("deltanet", **x, internals=True)
    e = np.array([3.0, -1.0]) / np.sqrt(10.0)
    np.testing.assert_allclose(h[0, 0, 0], e, rtol=1e-15)
    np.testing.assert_allclose(z[0, 0, 0], e, rtol=1e-15)
    np.testing.assert_allclose(o[0, 0, 0], [0.7, -1.3], rtol=1e-15)
    np.testing.assert_allclose(B_T[0, 0], np.outer([0.7, -1.3], e), rtol=1e-15)
    # a zero read makes a zero key: the second layer is left as it was
    x["A0"] = np.zeros((1, 1, 2, 2))
    x["B0"] = np.array([[0.5, 0.25], [-1.0, 2.0]]).reshape(1, 1, 2, 2)
    o, _, B_T, h, z = ttt_pre_fwd("deltanet", **x, internals=True)
    assert np.array_equal(h, np.zeros_like(h)) and np.array_equal(z, np.zeros_like(z))
    assert np.array_equal(B_T, x["B0"]) and np.array_equal(o, np.zeros_like(o))
