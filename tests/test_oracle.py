"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each pin checks the oracle against something fixed independently: values
worked by hand, exact rational arithmetic on the explicit transition-matrix
product, closed forms, reductions between the variants and invariants of the
update.  ``test_pins_catch_planted_mistakes`` plants plausible mistakes in a
copy of the oracle's recurrence and checks that some pin fails for each.
"""
import json
import os
from fractions import Fraction as F

import numpy as np
import pytest

import oracle.delta_oracle as od
from oracle import delta_decode, delta_fwd, efla_step_size, run_recurrence

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")


def _fr(x):
    return np.array([[F(e) for e in row] for row in x], dtype=object) if isinstance(x[0], list) \
        else np.array([F(e) for e in x], dtype=object)


def _rand_inputs(rng, variant, B, T, H, dk, dv, unit_k=True):
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    if unit_k:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, dv))
    if variant == "gdn2":
        beta = rng.uniform(0, 1, (B, T, H, dk))
        wgate = rng.uniform(0, 1, (B, T, H, dv))
    elif variant == "fg2":
        beta = rng.uniform(0, 1, (B, T, H, dk))
        wgate = None
    else:
        beta = rng.uniform(0, 1, (B, T, H))
        wgate = None
    g = {"deltanet": None,
         "gdn": -rng.uniform(0, 1, (B, T, H)),
         "kda": -rng.uniform(0, 1, (B, T, H, dk)),
         "gdn2": -rng.uniform(0, 1, (B, T, H, dk)),
         "fg2": -rng.uniform(0, 1, (B, T, H, dk))}[variant]
    S0 = 0.3 * rng.standard_normal((B, H, dv, dk))
    return dict(q=q, k=k, v=v, beta=beta, wgate=wgate, g=g, S0=S0)


# ---------------------------------------------------------------- pins


def pin_hand_worked():
    """Hand-derived two-channel examples (tests/golden/hand_worked.json)."""
    cases = json.load(open(GOLDEN))
    for name, case in cases.items():
        if name.startswith("_"):
            continue
        S = _fr(case["S0"])[None]
        toks = case["tokens"]
        T = len(toks)
        q = np.array([[_fr(t["q"]) for t in toks]], dtype=object)
        k = np.array([[_fr(t["k"]) for t in toks]], dtype=object)
        v = np.array([[_fr(t["v"]) for t in toks]], dtype=object)
        a = np.array([[_fr(t["a"]) for t in toks]], dtype=object)
        for t in range(1, T + 1):
            if case["variant"] == "gdn2":
                er = np.array([[_fr(x["erase"]) for x in toks[:t]]], dtype=object)
                wr = np.array([[_fr(x["write"]) for x in toks[:t]]], dtype=object)
                o, St = od.run_recurrence(S, q[:, :t], k[:, :t], v[:, :t], a[:, :t],
                                          erase=er, write=wr)
            else:
                be = np.array([[F(x["beta"]) for x in toks[:t]]], dtype=object)
                o, St = od.run_recurrence(S, q[:, :t], k[:, :t], v[:, :t], a[:, :t], beta=be)
            assert (St[0] == _fr(toks[t - 1]["S"])).all(), (name, t, St[0])
            assert (o[0, t - 1] == _fr(toks[t - 1]["o"])).all(), (name, t, o[0, t - 1])


def _mat(rows, cols, f):
    return [[f(i, j) for j in range(cols)] for i in range(rows)]


def _mm(A, B):
    return [[sum((A[i][m] * B[m][j] for m in range(len(B))), F(0)) for j in range(len(B[0]))]
            for i in range(len(A))]


def _madd(A, B):
    return [[A[i][j] + B[i][j] for j in range(len(A[0]))] for i in range(len(A))]


def pin_exact_product_form(seed=0):
    """Exact rationals: S_t = S_0 M_1..M_t + sum_s W_s M_{s+1}..M_t with explicit
    d_k×d_k transition matrices M_t = Diag(a_t)(I - beta_t k_t k_t^T) (split gates
    and FG^2-GDN: Diag(a_t)(I - k_t (b_t ⊙ k_t)^T)) and writes W_t = beta_t v_t k_t^T
    (split: (w_t ⊙ v_t) k_t^T; FG^2-GDN: v_t (b_t ⊙ k_t)^T), o_t = S_t q_t.  Must
    agree exactly."""
    rng = np.random.default_rng(seed)

    def rq(lo=-3, hi=4, den=(1, 2, 3, 4, 5)):
        return F(int(rng.integers(lo, hi)), int(rng.choice(den)))

    def rpos():
        return F(int(rng.integers(1, 6)), 5)   # in (0, 1]

    for variant in od.VARIANTS:
        for (T, dk, dv) in [(1, 2, 2), (4, 3, 2), (6, 2, 3)]:
            S0 = _mat(dv, dk, lambda i, j: rq())
            toks = []
            for _ in range(T):
                t = dict(q=[rq() for _ in range(dk)], k=[rq() for _ in range(dk)],
                         v=[rq() for _ in range(dv)])
                if variant == "deltanet":
                    t["a"] = [F(1)] * dk
                elif variant == "gdn":
                    t["a"] = [rpos()] * dk
                else:
                    t["a"] = [rpos() for _ in range(dk)]
                if variant == "gdn2":
                    t["b"] = [rpos() for _ in range(dk)]
                    t["w"] = [rpos() for _ in range(dv)]
                elif variant == "fg2":
                    t["b"] = [rpos() for _ in range(dk)]
                else:
                    t["beta"] = rpos()
                toks.append(t)
            Ms, Ws = [], []
            for t in toks:
                D = _mat(dk, dk, lambda i, j: t["a"][i] if i == j else F(0))
                if variant in ("gdn2", "fg2"):
                    E = _mat(dk, dk, lambda i, j: (F(1) if i == j else F(0))
                             - t["k"][i] * t["b"][j] * t["k"][j])
                    if variant == "gdn2":
                        Wt = _mat(dv, dk, lambda i, j: t["w"][i] * t["v"][i] * t["k"][j])
                    else:
                        Wt = _mat(dv, dk, lambda i, j: t["v"][i] * t["b"][j] * t["k"][j])
                else:
                    E = _mat(dk, dk, lambda i, j: (F(1) if i == j else F(0))
                             - t["beta"] * t["k"][i] * t["k"][j])
                    Wt = _mat(dv, dk, lambda i, j: t["beta"] * t["v"][i] * t["k"][j])
                Ms.append(_mm(D, E))
                Ws.append(Wt)
            o_ref = []
            for t in range(1, T + 1):
                St = S0
                for s in range(t):
                    St = _mm(St, Ms[s])
                for s in range(t):
                    term = Ws[s]
                    for u in range(s + 1, t):
                        term = _mm(term, Ms[u])
                    St = _madd(St, term)
                o_ref.append([sum((St[i][j] * toks[t - 1]["q"][j] for j in range(dk)), F(0))
                              for i in range(dv)])
            arr = lambda key: np.array([[t[key] for t in toks]], dtype=object)
            if variant == "gdn2":
                o, S_fin = od.run_recurrence(np.array([S0], dtype=object), arr("q"), arr("k"),
                                             arr("v"), arr("a"), erase=arr("b"), write=arr("w"))
            elif variant == "fg2":
                o, S_fin = od.run_recurrence(np.array([S0], dtype=object), arr("q"), arr("k"),
                                             arr("v"), arr("a"), keystep=arr("b"))
            else:
                o, S_fin = od.run_recurrence(np.array([S0], dtype=object), arr("q"), arr("k"),
                                             arr("v"), arr("a"), beta=arr("beta"))
            assert (S_fin[0] == np.array(St, dtype=object)).all(), (variant, T)
            assert (o[0] == np.array(o_ref, dtype=object)).all(), (variant, T)


def pin_beta_zero():
    """beta = 0 (split: b = w = 0) leaves only the decay: S_T = S_0 Diag(prod a_t)."""
    rng = np.random.default_rng(1)
    for variant in od.VARIANTS:
        x = _rand_inputs(rng, variant, 2, 7, 3, 5, 4)
        x["beta"] = np.zeros_like(x["beta"])
        if x["wgate"] is not None:
            x["wgate"] = np.zeros_like(x["wgate"])
        o, S = delta_fwd(variant, **x)
        if variant == "deltanet":
            decay = np.ones((2, 3, 5))
        elif variant == "gdn":
            decay = np.exp(x["g"].sum(axis=1))[..., None] * np.ones(5)
        else:
            decay = np.exp(x["g"].sum(axis=1))
        np.testing.assert_allclose(S, x["S0"] * decay[:, :, None, :], rtol=1e-13, atol=1e-15)
        if variant == "deltanet":
            assert np.array_equal(S, x["S0"])


def pin_gate_zero_is_deltanet():
    """Gated DeltaNet with g = 0 is DeltaNet, bitwise."""
    rng = np.random.default_rng(2)
    x = _rand_inputs(rng, "gdn", 2, 9, 2, 6, 5)
    o1, S1 = delta_fwd("gdn", **{**x, "g": np.zeros_like(x["g"])})
    o2, S2 = delta_fwd("deltanet", **{**x, "g": None})
    assert np.array_equal(o1, o2) and np.array_equal(S1, S2)


def pin_reductions():
    """KDA with a channel-constant decay is Gated DeltaNet; Gated DeltaNet-2 with
    b = beta·1 and w = beta·1 is KDA (Gated DeltaNet-2 abstract); FG^2-GDN with
    a channel-constant step size beta·1 is KDA (FG^2-GDN card: the vector
    generalises KDA's scalar step size)."""
    rng = np.random.default_rng(3)
    x = _rand_inputs(rng, "gdn", 2, 11, 3, 6, 5)
    o_gdn, S_gdn = delta_fwd("gdn", **x)
    g_vec = np.repeat(x["g"][..., None], 6, axis=-1)
    o_kda, S_kda = delta_fwd("kda", **{**x, "g": g_vec})
    np.testing.assert_allclose(o_kda, o_gdn, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(S_kda, S_gdn, rtol=1e-12, atol=1e-13)
    x = _rand_inputs(rng, "kda", 2, 11, 3, 6, 5)
    o_kda, S_kda = delta_fwd("kda", **x)
    b = np.repeat(x["beta"][..., None], 6, axis=-1)
    w = np.repeat(x["beta"][..., None], 5, axis=-1)
    o2, S2 = delta_fwd("gdn2", **{**x, "beta": b, "wgate": w})
    np.testing.assert_allclose(o2, o_kda, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(S2, S_kda, rtol=1e-12, atol=1e-13)
    o3, S3 = delta_fwd("fg2", **{**x, "beta": b})
    np.testing.assert_allclose(o3, o_kda, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(S3, S_kda, rtol=1e-12, atol=1e-13)


def pin_unit_write():
    """beta = 1 and unit k make the write exact: S_t k_t = v_t, and with q = k, o_t = v_t.
    Split gates with b = 1: S_t k_t = w_t ⊙ v_t."""
    rng = np.random.default_rng(4)
    for variant in od.VARIANTS:
        x = _rand_inputs(rng, variant, 2, 8, 2, 6, 6)
        x["beta"] = np.ones_like(x["beta"])
        x["q"] = x["k"]
        o, _ = delta_fwd(variant, **x)
        expect = x["v"] * (x["wgate"] if variant == "gdn2" else 1.0)
        np.testing.assert_allclose(o, expect, rtol=1e-12, atol=1e-12)
        # S_t k_t after token t: check on each prefix
        for t in (1, 5, 8):
            _, S = delta_fwd(variant, **{n: (None if a is None or n == "S0" else a[:, :t])
                                         for n, a in x.items() if n != "S0"}, S0=x["S0"])
            Sk = np.einsum("bhvk,bhk->bhv", S, x["k"][:, t - 1])
            np.testing.assert_allclose(Sk, expect[:, t - 1], rtol=1e-12, atol=1e-12)


def pin_orthonormal_keys():
    """k_t = e_t, S0 = 0: every read is zero and the rule is gated linear attention,
    o_t = sum_{s<=t} beta_s v_s q_t[s] prod_{u=s+1..t} a_u[s] (DeltaTTT summary, §2:
    evaluation at a fixed base gives additive linear attention)."""
    rng = np.random.default_rng(5)
    T, dk, dv = 6, 8, 3
    for variant in od.VARIANTS:
        x = _rand_inputs(rng, variant, 1, T, 1, dk, dv)
        k = np.zeros((1, T, 1, dk))
        for t in range(T):
            k[0, t, 0, t] = 1.0
        x["k"], x["S0"] = k, None
        o, _ = delta_fwd(variant, **x)
        if variant == "deltanet":
            a = np.ones((T, dk))
        elif variant == "gdn":
            a = np.exp(x["g"][0, :, 0])[:, None] * np.ones(dk)
        else:
            a = np.exp(x["g"][0, :, 0])
        exp = np.zeros((T, dv))
        for t in range(T):
            for s in range(t + 1):
                if variant == "gdn2":
                    wv = x["wgate"][0, s, 0] * x["v"][0, s, 0]
                elif variant == "fg2":   # the write along beta_s ⊙ e_s keeps channel s only
                    wv = x["beta"][0, s, 0, s] * x["v"][0, s, 0]
                else:
                    wv = x["beta"][0, s, 0] * x["v"][0, s, 0]
                exp[t] += wv * x["q"][0, t, 0, s] * np.prod(a[s + 1:t + 1, s])
        np.testing.assert_allclose(o[0, :, 0], exp, rtol=1e-12, atol=1e-14)


def pin_one_token_by_hand():
    """T = 1 with explicit matrices: S_1 = S_0 Diag(a)(I - beta k k^T) + beta v k^T."""
    rng = np.random.default_rng(6)
    x = _rand_inputs(rng, "kda", 1, 1, 1, 4, 3, unit_k=False)
    o, S = delta_fwd("kda", **x)
    k, v, q = x["k"][0, 0, 0], x["v"][0, 0, 0], x["q"][0, 0, 0]
    b, a = x["beta"][0, 0, 0], np.exp(x["g"][0, 0, 0])
    S1 = x["S0"][0, 0] @ np.diag(a) @ (np.eye(4) - b * np.outer(k, k)) + b * np.outer(v, k)
    np.testing.assert_allclose(S[0, 0], S1, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(o[0, 0, 0], S1 @ q, rtol=1e-13, atol=1e-14)


def pin_linearity():
    """For fixed q, k, gates, (v, S0) -> (o, S_T) is linear (the update is affine in the
    preceding memory, DeltaTTT summary §2)."""
    rng = np.random.default_rng(7)
    for variant in od.VARIANTS:
        x1 = _rand_inputs(rng, variant, 1, 9, 2, 5, 4)
        x2 = _rand_inputs(rng, variant, 1, 9, 2, 5, 4)
        for key in ("q", "k", "beta", "wgate", "g"):
            x2[key] = x1[key]
        c1, c2 = 0.7, -1.9
        mix = {**x1, "v": c1 * x1["v"] + c2 * x2["v"], "S0": c1 * x1["S0"] + c2 * x2["S0"]}
        o1, S1 = delta_fwd(variant, **x1)
        o2, S2 = delta_fwd(variant, **x2)
        om, Sm = delta_fwd(variant, **mix)
        np.testing.assert_allclose(om, c1 * o1 + c2 * o2, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(Sm, c1 * S1 + c2 * S2, rtol=1e-11, atol=1e-12)


def pin_norm_bound():
    """|k| = 1, beta in [0,1], a in (0,1]: ||S_t||_F <= ||S_{t-1}||_F + beta_t ||v_t||."""
    rng = np.random.default_rng(8)
    for variant in ("deltanet", "gdn", "kda"):
        x = _rand_inputs(rng, variant, 1, 12, 2, 5, 4)
        prev = np.linalg.norm(x["S0"], axis=(-2, -1))
        for t in range(1, 13):
            sl = {n: (None if a is None else a[:, :t]) for n, a in x.items() if n != "S0"}
            _, S = delta_fwd(variant, **sl, S0=x["S0"])
            cur = np.linalg.norm(S, axis=(-2, -1))
            bound = prev + x["beta"][:, t - 1] * np.linalg.norm(x["v"][:, t - 1], axis=-1)
            assert (cur <= bound + 1e-12).all()
            prev = cur


def pin_split_sequence():
    """Running 0:T1 then T1:T from the carried state equals running 0:T."""
    rng = np.random.default_rng(9)
    for variant in od.VARIANTS:
        x = _rand_inputs(rng, variant, 2, 13, 2, 4, 3)
        o, S = delta_fwd(variant, **x)
        cut = lambda a, s: None if a is None else a[:, s]
        per_tok = ("q", "k", "v", "beta", "wgate", "g")
        oa, Sa = delta_fwd(variant, **{n: cut(x[n], slice(0, 5)) for n in per_tok}, S0=x["S0"])
        ob, Sb = delta_fwd(variant, **{n: cut(x[n], slice(5, 13)) for n in per_tok}, S0=Sa)
        np.testing.assert_allclose(np.concatenate([oa, ob], axis=1), o, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(Sb, S, rtol=1e-12, atol=1e-13)


def pin_decode_is_one_token():
    rng = np.random.default_rng(10)
    for variant in od.VARIANTS:
        x = _rand_inputs(rng, variant, 3, 1, 2, 5, 4)
        o, S = delta_fwd(variant, **x)
        step = {n: (None if x[n] is None else x[n][:, 0]) for n in ("q", "k", "v", "beta", "wgate", "g")}
        od_, Sd = delta_decode(variant, **step, S=x["S0"])
        assert np.array_equal(od_, o[:, 0]) and np.array_equal(Sd, S)


def pin_grouped_heads_one_token():
    """4 value heads over 2 query/key heads, one token, written out per head: value
    head h reads the query and key of head h // 2 (Grouped Value Attention reading)."""
    rng = np.random.default_rng(11)
    B, H, Hk, dk, dv = 2, 4, 2, 5, 3
    q = rng.standard_normal((B, 1, Hk, dk))
    k = rng.standard_normal((B, 1, Hk, dk))
    v = rng.standard_normal((B, 1, H, dv))
    beta = rng.uniform(0, 1, (B, 1, H))
    g = -rng.uniform(0, 1, (B, 1, H))
    S0 = rng.standard_normal((B, H, dv, dk))
    o, S = delta_fwd("gdn", q, k, v, beta, g=g, S0=S0)
    assert o.shape == (B, 1, H, dv) and S.shape == (B, H, dv, dk)
    for b in range(B):
        for h in range(H):
            kk, qq = k[b, 0, h // 2], q[b, 0, h // 2]
            Sp = np.exp(g[b, 0, h]) * S0[b, h]
            S1 = Sp + beta[b, 0, h] * np.outer(v[b, 0, h] - Sp @ kk, kk)
            np.testing.assert_allclose(S[b, h], S1, rtol=1e-13, atol=1e-14)
            np.testing.assert_allclose(o[b, 0, h], S1 @ qq, rtol=1e-13, atol=1e-14)


def pin_grouped_heads_share():
    """Value heads of one group given the same v, gates and S0 produce the same outputs
    over a whole sequence; heads of different groups, given the same, do not."""
    rng = np.random.default_rng(12)
    for variant in od.VARIANTS:
        x = _rand_inputs(rng, variant, 1, 9, 6, 4, 3)
        G = 3   # 6 value heads over 2 query/key heads
        x["q"], x["k"] = x["q"][:, :, ::G], x["k"][:, :, ::G]
        for name in ("v", "beta", "wgate", "g"):
            if x[name] is not None:
                x[name][:, :, :] = x[name][:, :, :1]
        x["S0"][:, :] = x["S0"][:, :1]
        o, S = delta_fwd(variant, **x)
        for h in range(6):
            same = h // G == 0
            assert np.array_equal(o[:, :, h], o[:, :, 0]) == same, (variant, h)
            assert np.array_equal(S[:, h], S[:, 0]) == same, (variant, h)


def _rk4_flow(S, k, v, length, steps=400):
    """Integrate dS/dtau = (v - S k) k^T over [0, length] with classical RK4."""
    f = lambda X: np.outer(v - X @ k, k)  # noqa: E731
    h = length / steps
    for _ in range(steps):
        a1 = f(S)
        a2 = f(S + 0.5 * h * a1)
        a3 = f(S + 0.5 * h * a2)
        a4 = f(S + h * a3)
        S = S + h / 6 * (a1 + 2 * a2 + 2 * a3 + a4)
    return S


def pin_efla_exact_flow():
    """EFLA = the exact flow of dS/dtau = (v - S k) k^T over the length beta, after
    the decay: the oracle with efla_step_size matches an RK4 integration of that flow,
    token by token over a sequence, for key norms 0.3, 1 and 2.5."""
    rng = np.random.default_rng(13)
    dk, dv, T = 5, 3, 6
    for norm in (0.3, 1.0, 2.5):
        q = rng.standard_normal((1, T, 1, dk))
        k = rng.standard_normal((1, T, 1, dk))
        k *= norm / np.linalg.norm(k, axis=-1, keepdims=True)
        v = rng.standard_normal((1, T, 1, dv))
        beta = rng.uniform(0.2, 1, (1, T, 1))
        g = -rng.uniform(0, 1, (1, T, 1))
        S0 = rng.standard_normal((1, 1, dv, dk))
        o, S_T = delta_fwd("gdn", q, k, v, efla_step_size(k, beta), g=g, S0=S0)
        S = S0[0, 0]
        for t in range(T):
            S = _rk4_flow(np.exp(g[0, t, 0]) * S, k[0, t, 0], v[0, t, 0], beta[0, t, 0])
            np.testing.assert_allclose(o[0, t, 0], S @ q[0, t, 0], rtol=1e-9, atol=1e-11)
        np.testing.assert_allclose(S_T[0, 0], S, rtol=1e-9, atol=1e-11)


def pin_efla_limits():
    """k = 0 gives beta; |k| = 1 gives 1 - e^{-beta}; beta |k|^2 -> 0 gives beta to first
    order; in general 0 < c <= min(beta, 1 / |k|^2).  Grouped heads share the norm."""
    beta = np.array([[0.0, 0.3, 1.0, 5.0]])
    zero = np.zeros((1, 1, 3))
    np.testing.assert_array_equal(efla_step_size(zero, beta), beta)
    unit = np.array([[[0.6, 0.8, 0.0]]])
    np.testing.assert_allclose(efla_step_size(unit, beta), 1 - np.exp(-beta), rtol=1e-15)
    tiny = np.array([[[1e-9, 0.0, 0.0]]])
    np.testing.assert_allclose(efla_step_size(tiny, beta), beta, rtol=1e-15)
    rng = np.random.default_rng(14)
    k = rng.standard_normal((3, 7, 2, 4)) * rng.uniform(0.1, 4, (3, 7, 2, 1))
    b = rng.uniform(0.01, 2, (3, 7, 6))
    c = efla_step_size(k, b)
    kappa = np.repeat(np.sum(k * k, axis=-1), 3, axis=-1)
    assert (c > 0).all() and (c <= b).all() and (c <= 1 / kappa + 1e-15).all()
    for h in range(6):   # value head h reads key head h // 3
        kap = np.sum(k[..., h // 3, :] ** 2, axis=-1)
        np.testing.assert_allclose(c[..., h], -np.expm1(-b[..., h] * kap) / kap, rtol=1e-14)


def pin_fg2_per_coordinate_step():
    """One FG^2-GDN token is one gradient step on L(S) = 1/2 ||S k - v||^2 from the
    decayed state S' with its own step size per key channel (FG^2-GDN card: per-
    coordinate step sizes as in AdaGrad/Adam): S_1 = S' - (dL/dS at S') Diag(beta),
    o = S_1 q.  The gradient is taken by central differences, which are exact for a
    quadratic up to rounding, so the formula of the update is not retyped here."""
    rng = np.random.default_rng(12)
    dk, dv = 5, 4
    x = _rand_inputs(rng, "fg2", 1, 1, 1, dk, dv, unit_k=False)
    o, S = delta_fwd("fg2", **x)
    Sp = x["S0"][0, 0] * np.exp(x["g"][0, 0, 0])[None, :]
    k, v = x["k"][0, 0, 0], x["v"][0, 0, 0]

    def loss(M):
        r = M @ k - v
        return 0.5 * float(r @ r)

    grad = np.zeros((dv, dk))
    h = 1e-3
    for i in range(dv):
        for j in range(dk):
            E = np.zeros((dv, dk))
            E[i, j] = h
            grad[i, j] = (loss(Sp + E) - loss(Sp - E)) / (2 * h)
    expect = Sp - grad * x["beta"][0, 0, 0][None, :]
    np.testing.assert_allclose(S[0, 0], expect, rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(o[0, 0, 0], expect @ x["q"][0, 0, 0], rtol=1e-9, atol=1e-11)


PINS = [pin_hand_worked, pin_exact_product_form, pin_beta_zero, pin_gate_zero_is_deltanet,
        pin_reductions, pin_unit_write, pin_orthonormal_keys, pin_one_token_by_hand,
        pin_linearity, pin_norm_bound, pin_split_sequence, pin_decode_is_one_token,
        pin_grouped_heads_one_token, pin_grouped_heads_share, pin_efla_exact_flow,
        pin_efla_limits, pin_fg2_per_coordinate_step]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin()


# ------------------------------------------------- planted mistakes


def _mutant(kind):
    """A copy of the oracle's recurrence with one plausible mistake planted."""

    def rec(S0, q, k, v, a, beta=None, erase=None, write=None, keystep=None):
        split = erase is not None
        S = np.array(S0, copy=True)
        N, T, _ = q.shape
        o = np.empty((N, T, v.shape[2]), dtype=S.dtype)
        for t in range(T):
            kt = k[:, t, :]
            Sp = S * a[:, t, None, :]
            if kind == "decay_after_read":
                r = (S @ kt[:, :, None])[:, :, 0]
            elif kind == "decay_rows":
                Sp = S * a[:, t, :, None] if S.shape[1] == S.shape[2] else Sp
                r = (Sp @ kt[:, :, None])[:, :, 0]
            else:
                r = (Sp @ kt[:, :, None])[:, :, 0]
            if split:
                ek = erase[:, t, :] * kt
                if kind == "erase_swapped":
                    upd = -(Sp @ ek[:, :, None]) * kt[:, None, :]
                else:
                    upd = -r[:, :, None] * ek[:, None, :]
                wv = write[:, t, :] * v[:, t, :]
                if kind == "write_gate_dropped":
                    wv = v[:, t, :]
                Snew = Sp + upd + wv[:, :, None] * kt[:, None, :]
            elif keystep is not None:
                ek = keystep[:, t, :] * kt
                res = v[:, t, :] - r
                if kind == "sign":
                    res = v[:, t, :] + r
                if kind == "keystep_write_along_k":
                    Snew = Sp - r[:, :, None] * ek[:, None, :] + v[:, t, :, None] * kt[:, None, :]
                elif kind == "keystep_read_scaled":
                    res = v[:, t, :] - (Sp @ ek[:, :, None])[:, :, 0]
                    Snew = Sp + res[:, :, None] * ek[:, None, :]
                else:
                    Snew = Sp + res[:, :, None] * ek[:, None, :]
            else:
                res = v[:, t, :] - r
                if kind == "sign":
                    res = v[:, t, :] + r
                if kind == "beta_dropped_on_read":
                    res = beta[:, t, None] * v[:, t, :] - r
                    Snew = Sp + res[:, :, None] * kt[:, None, :]
                else:
                    Snew = Sp + beta[:, t, None, None] * res[:, :, None] * kt[:, None, :]
                if kind == "transposed_write" and S.shape[1] == S.shape[2]:
                    Snew = Sp + beta[:, t, None, None] * kt[:, :, None] * res[:, None, :]
            if kind == "readout_before_write":
                o[:, t, :] = (S @ q[:, t, :, None])[:, :, 0]
            elif kind == "readout_decayed_only":
                o[:, t, :] = (Sp @ q[:, t, :, None])[:, :, 0]
            else:
                o[:, t, :] = (Snew @ q[:, t, :, None])[:, :, 0]
            S = Snew
        return o, S

    return rec


MUTANTS = ["decay_after_read", "decay_rows", "erase_swapped", "write_gate_dropped", "sign",
           "beta_dropped_on_read", "transposed_write", "readout_before_write",
           "readout_decayed_only", "keystep_write_along_k", "keystep_read_scaled"]


@pytest.mark.parametrize("kind", MUTANTS)
def test_pins_catch_planted_mistakes(kind, monkeypatch):
    monkeypatch.setattr(od, "run_recurrence", _mutant(kind))
    failed = []
    for pin in PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError) as e:  # noqa: PERF203
            failed.append(pin.__name__)
    assert failed, f"no pin caught the planted mistake {kind!r}"


def test_unmutated_copy_passes(monkeypatch):
    """The mutant factory without a mistake must pass every pin (guards the test above)."""
    monkeypatch.setattr(od, "run_recurrence", _mutant("none"))
    for pin in PINS:
        pin()
