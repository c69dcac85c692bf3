"""Pins of the oracle's backward pass (reverse mode of the token recurrence).

Two independent checks, neither of which uses the oracle's backward code:
  * central finite differences of L = <dO, o> + <dS_T, S_T> through the oracle's
    forward (itself pinned in test_oracle.py), along random directions, for every
    input of every variant, including grouped query/key heads;
  * torch.autograd in float64 on the CPU through a separate, direct torch
    transcription of the recurrence.
"""
import numpy as np
import pytest
import torch

from oracle import delta_bwd, delta_fwd

VARIANTS = ["deltanet", "gdn", "kda", "gdn2", "fg2"]


def _inputs(rng, variant, B=2, T=7, H=2, Hk=None, dk=4, dv=3):
    Hk = H if Hk is None else Hk
    x = dict(q=rng.standard_normal((B, T, Hk, dk)), k=rng.standard_normal((B, T, Hk, dk)) * 0.6,
             v=rng.standard_normal((B, T, H, dv)), S0=rng.standard_normal((B, H, dv, dk)) * 0.5)
    if variant == "gdn2":
        x["beta"] = rng.uniform(0.1, 0.9, (B, T, H, dk))
        x["wgate"] = rng.uniform(0.1, 0.9, (B, T, H, dv))
    elif variant == "fg2":
        x["beta"] = rng.uniform(0.1, 0.9, (B, T, H, dk))
        x["wgate"] = None
    else:
        x["beta"] = rng.uniform(0.1, 0.9, (B, T, H))
        x["wgate"] = None
    x["g"] = {"deltanet": None, "gdn": -rng.uniform(0, 1, (B, T, H)),
              "kda": -rng.uniform(0, 1, (B, T, H, dk)),
              "gdn2": -rng.uniform(0, 1, (B, T, H, dk)),
              "fg2": -rng.uniform(0, 1, (B, T, H, dk))}[variant]
    dO = rng.standard_normal((B, T, H, dv))
    dST = rng.standard_normal((B, H, dv, dk))
    return x, dO, dST


def _loss(variant, x, dO, dST):
    o, S = delta_fwd(variant, **x)
    return float(np.sum(o * dO) + np.sum(S * dST))


GRAD_OF = {"q": "dq", "k": "dk", "v": "dv", "beta": "dbeta", "wgate": "dwgate", "g": "dg",
           "S0": "dS0"}


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("Hk", [2, 1])
def test_finite_differences(variant, Hk):
    rng = np.random.default_rng(100 + VARIANTS.index(variant) + 10 * Hk)
    x, dO, dST = _inputs(rng, variant, Hk=Hk)
    grads = delta_bwd(variant, **x, dO=dO, dS_T=dST)
    eps = 1e-6
    for name, gname in GRAD_OF.items():
        if x[name] is None:
            assert grads[gname] is None
            continue
        for _ in range(3):
            d = rng.standard_normal(x[name].shape)
            xp = {**x, name: x[name] + eps * d}
            xm = {**x, name: x[name] - eps * d}
            num = (_loss(variant, xp, dO, dST) - _loss(variant, xm, dO, dST)) / (2 * eps)
            ana = float(np.sum(grads[gname] * d))
            assert abs(num - ana) <= 1e-6 * max(1.0, abs(ana)), (name, num, ana)


def _torch_forward(variant, x):
    """Direct transcription of the token update in torch (independent of the oracle)."""
    q, k, v, S = x["q"], x["k"], x["v"], x["S0"]
    B, T, H, dv = v.shape
    G = H // q.shape[2]
    q = q.repeat_interleave(G, dim=2)
    k = k.repeat_interleave(G, dim=2)
    outs = []
    for t in range(T):
        kt, qt, vt = k[:, t], q[:, t], v[:, t]                    # [B, H, d]
        if variant == "deltanet":
            a = torch.ones_like(kt)
        elif variant == "gdn":
            a = torch.exp(x["g"][:, t])[..., None].expand_as(kt)
        else:
            a = torch.exp(x["g"][:, t])
        Sp = S * a[:, :, None, :]
        r = torch.einsum("bhij,bhj->bhi", Sp, kt)
        if variant == "gdn2":
            S = (Sp - r[..., :, None] * (x["beta"][:, t] * kt)[..., None, :]
                 + (x["wgate"][:, t] * vt)[..., :, None] * kt[..., None, :])
        elif variant == "fg2":
            S = Sp + (vt - r)[..., :, None] * (x["beta"][:, t] * kt)[..., None, :]
        else:
            S = Sp + x["beta"][:, t][..., None, None] * (vt - r)[..., :, None] * kt[..., None, :]
        outs.append(torch.einsum("bhij,bhj->bhi", S, qt))
    return torch.stack(outs, dim=1), S


@pytest.mark.parametrize("variant", VARIANTS)
def test_torch_autograd(variant):
    rng = np.random.default_rng(200 + VARIANTS.index(variant))
    x, dO, dST = _inputs(rng, variant, B=2, T=9, H=4, Hk=2, dk=5, dv=3)
    xt = {n: (None if a is None else torch.tensor(a, dtype=torch.float64, requires_grad=True))
          for n, a in x.items()}
    o, S = _torch_forward(variant, xt)
    L = (o * torch.tensor(dO)).sum() + (S * torch.tensor(dST)).sum()
    L.backward()
    grads = delta_bwd(variant, **x, dO=dO, dS_T=dST)
    for name, gname in GRAD_OF.items():
        if xt[name] is None:
            continue
        np.testing.assert_allclose(grads[gname], xt[name].grad.numpy(), rtol=1e-10, atol=1e-12,
                                   err_msg=name)


def test_zero_upstream_gives_zero_gradients():
    rng = np.random.default_rng(300)
    x, dO, dST = _inputs(rng, "kda")
    grads = delta_bwd("kda", **x, dO=np.zeros_like(dO), dS_T=None)
    for gname in ("dq", "dk", "dv", "dbeta", "dg", "dS0"):
        assert not np.any(grads[gname]), gname
