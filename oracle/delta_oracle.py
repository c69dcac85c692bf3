"""CPU oracle for the gated delta-rule recurrence (token by token, float64).

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The product
path never calls it, and it shares no code with the HIP kernels.

What it computes is the plain definition of the recurrence, one token at a
time, on the exact (already rounded) input values the GPU receives:

* the delta rule is one serial gradient step of a linear memory on the
  regression loss 1/2 ||S k - v||^2: read ``S k``, subtract it from the
  value, write the residual along ``k`` with step size beta (DeltaTTT
  summary, paperlayer.ai, §2 Background and §4.1 "Layerwise memory
  optimization"; Gated DeltaNet-2 abstract, thelatestinai.com/papers/2607.07953:
  delta-rule models subtract the current read before writing a new value);
* a decay multiplies the memory before the read: a scalar per head and token
  for Gated DeltaNet, a vector over key channels for Kimi Delta Attention
  ("Delta-Rule Linear Attention" topic page, FG^2-GDN card: KDA refines the
  head-wise decay gate into channel-wise decay);
* Gated DeltaNet-2 replaces the single step size by a channel-wise erase gate
  b (key side) and a channel-wise write gate w (value side), and reduces to
  KDA when both equal the same scalar (Gated DeltaNet-2 abstract);
* FG^2-GDN ("Delta-Rule Linear Attention" topic page, FG^2-GDN card) turns the
  scalar step size of KDA into a channel-wise vector, as a per-coordinate
  optimizer turns one learning rate into one per coordinate.  Reading: the
  coordinates are the key channels, so the step is the gradient of
  1/2 ||S' k - v||^2, which is (S' k - v) k^T, scaled column by column by
  beta_t: the residual is written along beta_t ⊙ k_t.  The card's FG^2-GDN+
  (separate erase and write scales for keys and values) is the split-gate
  form above.

With S of shape [d_v, d_k] and a_t the decay (1, a scalar, or a d_k-vector),
one token does, in this order:

    S'  = S · Diag(a_t)                          decay the key columns
    r   = S' k_t                                  read
    S   = S' + beta_t (v_t - r) k_t^T             DeltaNet, GDN, KDA
    S   = S' - r (b_t ⊙ k_t)^T + (w_t ⊙ v_t) k_t^T   Gated DeltaNet-2
    S   = S' + (v_t - r) (beta_t ⊙ k_t)^T         FG^2-GDN (beta_t a d_k-vector)
    o_t = S q_t                                   readout after the write

The erase placement ``r (b ⊙ k)^T`` for Gated DeltaNet-2 is a reading: the
abstract names the two gates but prints no formula.  That reading is parity
unpinned beyond the reduction to KDA at b = w = beta.  The FG^2-GDN reading is
pinned to the per-coordinate gradient step it is named after and to its
reduction to KDA at beta_t = beta·1; which axis carries the vector is the
reading.

Two further forms from the same topic page:

* Grouped Value Attention (GDN FPGA decode card): fewer query/key heads than
  value heads.  Reading: with H value heads and H_k query/key heads, value
  head h uses query/key head h // (H / H_k), so consecutive value heads form
  a group; each value head keeps its own state, step size and decay.
* EFLA (EFLA card): the delta-rule write is an explicit Euler step of the flow
  dS/dtau = (v - S k) k^T over a length beta; EFLA takes the exact flow
  instead.  ``efla_step_size`` gives the step size that makes one delta-rule
  write equal that flow (derived in its docstring); the decay is applied
  before the flow, as before the write (a reading: the card names no gate).

``run_recurrence`` works on any numpy dtype, including ``object`` arrays of
``fractions.Fraction`` for exact-arithmetic tests; the public wrappers use
float64.
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

VARIANTS = ("deltanet", "gdn", "kda", "gdn2", "fg2")


def run_recurrence(S0: np.ndarray, q: np.ndarray, k: np.ndarray, v: np.ndarray,
                   a: np.ndarray, beta: Optional[np.ndarray] = None,
                   erase: Optional[np.ndarray] = None, write: Optional[np.ndarray] = None,
                   keystep: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Sequential recurrence over a batch of independent sequences.

    S0: [N, dv, dk]; q, k: [N, T, dk]; v: [N, T, dv]; a: [N, T, dk] decay
    factors (already broadcast over key channels).  Exactly one of: ``beta``
    [N, T] (single step size), both ``erase`` [N, T, dk] and ``write``
    [N, T, dv] (split gates), or ``keystep`` [N, T, dk] (a step size per key
    channel, FG^2-GDN).  Returns o [N, T, dv] and the final state [N, dv, dk].
    """
    split = erase is not None
    modes = (beta is not None) + split + (keystep is not None)
    if split != (write is not None) or modes != 1:
        raise ValueError("pass either beta, or both erase and write, or keystep")
    S = np.array(S0, copy=True)
    N, T, _ = q.shape
    o = np.empty((N, T, v.shape[2]), dtype=S.dtype)
    for t in range(T):
        kt = k[:, t, :]
        Sp = S * a[:, t, None, :]
        r = (Sp @ kt[:, :, None])[:, :, 0]
        if split:
            S = (Sp - r[:, :, None] * (erase[:, t, :] * kt)[:, None, :]
                 + (write[:, t, :] * v[:, t, :])[:, :, None] * kt[:, None, :])
        elif keystep is not None:
            S = Sp + (v[:, t, :] - r)[:, :, None] * (keystep[:, t, :] * kt)[:, None, :]
        else:
            S = Sp + beta[:, t, None, None] * (v[:, t, :] - r)[:, :, None] * kt[:, None, :]
        o[:, t, :] = (S @ q[:, t, :, None])[:, :, 0]
    return o, S


def _decay(variant: str, g: Optional[np.ndarray], lead: tuple, dk: int) -> np.ndarray:
    """Per-channel decay factors a = exp(g), broadcast to lead + (dk,)."""
    if variant == "deltanet":
        if g is not None:
            raise ValueError("the ungated form takes no decay")
        return np.ones(lead + (dk,), dtype=np.float64)
    if g is None:
        raise ValueError(f"{variant} needs a log-decay")
    g = np.asarray(g, dtype=np.float64)
    if variant == "gdn":
        if g.shape != lead:
            raise ValueError(f"scalar decay must have shape {lead}, got {g.shape}")
        return np.broadcast_to(np.exp(g)[..., None], lead + (dk,))
    if g.shape != lead + (dk,):
        raise ValueError(f"channel decay must have shape {lead + (dk,)}, got {g.shape}")
    return np.exp(g)


def _to_heads(x: Optional[np.ndarray]) -> Optional[np.ndarray]:
    """[B, T, H, ...] -> [B*H, T, ...] in float64."""
    if x is None:
        return None
    x = np.asarray(x, dtype=np.float64)
    B, T, H = x.shape[:3]
    x = np.moveaxis(x, 2, 1)
    return x.reshape((B * H, T) + x.shape[3:])


def group_heads(x: np.ndarray, H: int) -> np.ndarray:
    """Query/key tensor [B, T, H_k, d] -> [B, T, H, d]: value head h reads
    query/key head h // (H / H_k) (Grouped Value Attention, reading above)."""
    Hk = x.shape[2]
    if Hk < 1 or H % Hk != 0:
        raise ValueError(f"{Hk} query/key heads do not divide {H} value heads")
    return np.repeat(x, H // Hk, axis=2)


def efla_step_size(k, beta) -> np.ndarray:
    """EFLA step size per value head, float64.

    k: [B, T, H_k, dk] (or [B, H_k, dk]); beta: [B, T, H] (or [B, H]).

    With kappa = |k|^2 and M = k k^T (eigenvalue kappa along k, 0 across it),
    exp(-u M) = I - (1 - e^{-u kappa}) / kappa * M, so k^T exp(-u M) =
    e^{-u kappa} k^T.  The flow of dS/dtau = (v - S k) k^T = -S M + v k^T from
    S' over a length beta is

        S' exp(-beta M) + int_0^beta v k^T exp(-(beta - s) M) ds
          = S' - c (S' k) k^T + c v k^T,   c = (1 - e^{-beta kappa}) / kappa,

    a delta-rule write with step size c (c -> beta as kappa -> 0).
    """
    k = np.asarray(k, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    kappa = np.sum(k * k, axis=-1)
    H = beta.shape[-1]
    Hk = kappa.shape[-1]
    if H % Hk != 0:
        raise ValueError(f"{Hk} query/key heads do not divide {H} value heads")
    kappa = np.repeat(kappa, H // Hk, axis=-1)
    safe = np.where(kappa > 0, kappa, 1.0)
    return np.where(kappa > 0, -np.expm1(-beta * kappa) / safe, beta)


def delta_fwd(variant: str, q, k, v, beta=None, wgate=None, g=None, S0=None
              ) -> Tuple[np.ndarray, np.ndarray]:
    """Forward pass over a whole sequence, argument layout of the C boundary.

    q, k: [B, T, H_k, dk] with H_k dividing H (H_k = H unless the value heads
    are grouped); v: [B, T, H, dv]; beta: [B, T, H] (for gdn2 the erase
    gate, for fg2 the channel-wise step size: [B, T, H, dk]); wgate: gdn2
    write gate [B, T, H, dv], else None;
    g: log-decay, None / [B, T, H] / [B, T, H, dk]; S0: [B, H, dv, dk] or None
    (zero state).  Returns o [B, T, H, dv] and S_T [B, H, dv, dk], float64.
    """
    if variant not in VARIANTS:
        raise ValueError(f"unknown variant {variant!r}")
    B, T, H, dv = np.shape(v)
    q = group_heads(np.asarray(q, dtype=np.float64), H)
    k = group_heads(np.asarray(k, dtype=np.float64), H)
    dk = q.shape[3]
    a = _to_heads(_decay(variant, g, (B, T, H), dk))
    if S0 is None:
        S = np.zeros((B * H, dv, dk), dtype=np.float64)
    else:
        S = np.asarray(S0, dtype=np.float64).reshape(B * H, dv, dk)
    if variant == "gdn2":
        if wgate is None:
            raise ValueError("gdn2 needs the write gate")
        o, S = run_recurrence(S, _to_heads(q), _to_heads(k), _to_heads(v), a,
                              erase=_to_heads(beta), write=_to_heads(wgate))
    elif variant == "fg2":
        if wgate is not None:
            raise ValueError("only gdn2 takes a write gate")
        if np.shape(beta) != (B, T, H, dk):
            raise ValueError(f"fg2 step sizes must have shape {(B, T, H, dk)}")
        o, S = run_recurrence(S, _to_heads(q), _to_heads(k), _to_heads(v), a,
                              keystep=_to_heads(beta))
    else:
        if wgate is not None:
            raise ValueError("only gdn2 takes a write gate")
        o, S = run_recurrence(S, _to_heads(q), _to_heads(k), _to_heads(v), a,
                              beta=_to_heads(beta))
    o = np.moveaxis(o.reshape(B, H, T, dv), 1, 2)
    return np.ascontiguousarray(o), S.reshape(B, H, dv, dk)


def delta_decode(variant: str, q, k, v, beta=None, wgate=None, g=None, S=None
                 ) -> Tuple[np.ndarray, np.ndarray]:
    """One decode step: per-token tensors [B, H, d] (q, k [B, H_k, dk]; beta/g
    [B, H] or [B, H, dk]), state S [B, H, dv, dk].  Returns o [B, H, dv] and the new state, float64."""
    add_t = (lambda x: None if x is None else np.asarray(x)[:, None])
    o, S_new = delta_fwd(variant, add_t(q), add_t(k), add_t(v), add_t(beta), add_t(wgate),
                         add_t(g), S)
    return o[:, 0], S_new


def _recurrence_backward(S0, q, k, v, a, dO, dST, beta=None, erase=None, write=None, keystep=None):
    """Reverse mode of ``run_recurrence`` (same argument layout, float64).

    Runs the recurrence forward keeping every state, then walks back one token
    at a time applying the chain rule to each line of the token update (order
    of the module docstring).  ``dO`` [N, T, dv] and ``dST`` [N, dv, dk] (or
    None) are the gradients arriving at o and at the final state.  Returns a
    dict with dq, dk, dv [N, T, d], da [N, T, dk] (gradient of the decay
    factors), dbeta [N, T] or (derase [N, T, dk], dwrite [N, T, dv]) or
    dkeystep [N, T, dk], and dS0.
    """
    split = erase is not None
    N, T, dk = q.shape
    S = np.array(S0, dtype=np.float64, copy=True)
    states = [S]
    for t in range(T):
        kt = k[:, t, :]
        Sp = S * a[:, t, None, :]
        r = (Sp @ kt[:, :, None])[:, :, 0]
        if split:
            S = (Sp - r[:, :, None] * (erase[:, t, :] * kt)[:, None, :]
                 + (write[:, t, :] * v[:, t, :])[:, :, None] * kt[:, None, :])
        elif keystep is not None:
            S = Sp + (v[:, t, :] - r)[:, :, None] * (keystep[:, t, :] * kt)[:, None, :]
        else:
            S = Sp + beta[:, t, None, None] * (v[:, t, :] - r)[:, :, None] * kt[:, None, :]
        states.append(S)
    lam = np.zeros_like(S) if dST is None else np.array(dST, dtype=np.float64, copy=True)
    g = {name: np.zeros_like(x) for name, x in (("dq", q), ("dk", k), ("dv", v), ("da", a))}
    if split:
        g["derase"] = np.zeros_like(erase)
        g["dwrite"] = np.zeros_like(write)
    elif keystep is not None:
        g["dkeystep"] = np.zeros_like(keystep)
    else:
        g["dbeta"] = np.zeros_like(beta)
    for t in range(T - 1, -1, -1):
        kt, qt, vt = k[:, t, :], q[:, t, :], v[:, t, :]
        S_prev, S_t = states[t], states[t + 1]
        Sp = S_prev * a[:, t, None, :]
        r = (Sp @ kt[:, :, None])[:, :, 0]
        # o_t = S_t q_t
        lam = lam + dO[:, t, :, None] * qt[:, None, :]
        g["dq"][:, t] = (np.swapaxes(S_t, 1, 2) @ dO[:, t, :, None])[:, :, 0]
        lam_k = (lam @ kt[:, :, None])[:, :, 0]                       # Λ k        [N, dv]
        if split:
            # S_t = S' - r (b ⊙ k)^T + (w ⊙ v) k^T
            eb = erase[:, t, :] * kt
            lamT_r = (np.swapaxes(lam, 1, 2) @ r[:, :, None])[:, :, 0]  # Λ^T r      [N, dk]
            wv = write[:, t, :] * vt
            g["derase"][:, t] = -lamT_r * kt
            g["dwrite"][:, t] = lam_k * vt
            g["dv"][:, t] = lam_k * write[:, t, :]
            dk_t = -lamT_r * erase[:, t, :] + (np.swapaxes(lam, 1, 2) @ wv[:, :, None])[:, :, 0]
            dr = -(lam @ eb[:, :, None])[:, :, 0]
        elif keystep is not None:
            # S_t = S' + u e^T with u = v - r, e = beta ⊙ k (beta per key channel)
            ek = keystep[:, t, :] * kt
            u = vt - r
            lam_e = (lam @ ek[:, :, None])[:, :, 0]                    # Λ e        [N, dv]
            de = (np.swapaxes(lam, 1, 2) @ u[:, :, None])[:, :, 0]     # Λ^T u      [N, dk]
            g["dkeystep"][:, t] = de * kt
            g["dv"][:, t] = lam_e
            dk_t = de * keystep[:, t, :]
            dr = -lam_e
        else:
            # S_t = S' + u k^T with u = beta (v - r)
            e = vt - r
            u = beta[:, t, None] * e
            g["dbeta"][:, t] = np.sum(lam_k * e, axis=1)
            g["dv"][:, t] = beta[:, t, None] * lam_k
            dk_t = (np.swapaxes(lam, 1, 2) @ u[:, :, None])[:, :, 0]
            dr = -beta[:, t, None] * lam_k
        # r = S' k: adds dr k^T to dS' and S'^T dr to dk
        dSp = lam + dr[:, :, None] * kt[:, None, :]
        g["dk"][:, t] = dk_t + (np.swapaxes(Sp, 1, 2) @ dr[:, :, None])[:, :, 0]
        # S' = S_prev Diag(a_t)
        g["da"][:, t] = np.sum(S_prev * dSp, axis=1)
        lam = dSp * a[:, t, None, :]
    g["dS0"] = lam
    return g


def _from_heads(x: np.ndarray, B: int, H: int) -> np.ndarray:
    """[B*H, T, ...] -> [B, T, H, ...]."""
    x = x.reshape((B, H) + x.shape[1:])
    return np.ascontiguousarray(np.moveaxis(x, 1, 2))


def delta_bwd(variant: str, q, k, v, beta=None, wgate=None, g=None, S0=None, dO=None, dS_T=None
              ) -> dict:
    """Gradients of the forward pass, float64, argument layout of delta_fwd.

    Given the gradient ``dO`` [B, T, H, dv] arriving at o and ``dS_T``
    [B, H, dv, dk] (None = zero) arriving at the final state, returns a dict
    with dq, dk (of the query/key heads given, summed over each group of value
    heads), dv, dbeta (for gdn2 the erase-gate gradient [B, T, H, dk]),
    dwgate (gdn2 only, else None), dg (None for deltanet; [B, T, H] for gdn,
    [B, T, H, dk] for kda/gdn2) and dS0 [B, H, dv, dk].  The decay factor is
    a = exp(g), so dg = a * dL/da per channel, summed over channels for gdn.
    """
    if variant not in VARIANTS:
        raise ValueError(f"unknown variant {variant!r}")
    B, T, H, dv = np.shape(v)
    q0 = np.asarray(q, dtype=np.float64)
    Hk = q0.shape[2]
    qh = _to_heads(group_heads(q0, H))
    kh = _to_heads(group_heads(np.asarray(k, dtype=np.float64), H))
    dk_ = qh.shape[2]
    a = _to_heads(_decay(variant, g, (B, T, H), dk_))
    S = (np.zeros((B * H, dv, dk_)) if S0 is None
         else np.asarray(S0, dtype=np.float64).reshape(B * H, dv, dk_))
    dST = None if dS_T is None else np.asarray(dS_T, dtype=np.float64).reshape(B * H, dv, dk_)
    dOh = _to_heads(dO)
    if variant == "gdn2":
        gr = _recurrence_backward(S, qh, kh, _to_heads(v), a, dOh, dST,
                                  erase=_to_heads(beta), write=_to_heads(wgate))
    elif variant == "fg2":
        gr = _recurrence_backward(S, qh, kh, _to_heads(v), a, dOh, dST, keystep=_to_heads(beta))
    else:
        gr = _recurrence_backward(S, qh, kh, _to_heads(v), a, dOh, dST, beta=_to_heads(beta))

    def ungroup(x):   # [B, T, H, d] -> sum over each group of value heads -> [B, T, Hk, d]
        return x.reshape(B, T, Hk, H // Hk, -1).sum(axis=3)

    out = {"dq": ungroup(_from_heads(gr["dq"], B, H)), "dk": ungroup(_from_heads(gr["dk"], B, H)),
           "dv": _from_heads(gr["dv"], B, H), "dwgate": None, "dg": None,
           "dS0": gr["dS0"].reshape(B, H, dv, dk_)}
    if variant == "gdn2":
        out["dbeta"] = _from_heads(gr["derase"], B, H)
        out["dwgate"] = _from_heads(gr["dwrite"], B, H)
    elif variant == "fg2":
        out["dbeta"] = _from_heads(gr["dkeystep"], B, H)
    else:
        out["dbeta"] = _from_heads(gr["dbeta"], B, H)
    if variant != "deltanet":
        dgc = _from_heads(gr["da"] * a, B, H)          # d/dg of exp(g), per channel
        out["dg"] = dgc.sum(axis=-1) if variant == "gdn" else dgc
    return out


# ------------------------------------------------------------------ DeltaTTT-pre


def _silu(x: np.ndarray) -> np.ndarray:
    return x / (1.0 + np.exp(-x))


def _unit_rows(x: np.ndarray) -> np.ndarray:
    """x / ||x|| over the last axis; a zero vector stays zero."""
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return np.where(n > 0, x / np.where(n > 0, n, 1.0), 0.0)


def ttt_pre_fwd(variant: str, q, k, v, beta1, g1=None, beta2=None, g2=None, A0=None, B0=None,
                internals: bool = False):
    """DeltaTTT-pre: a two-layer memory whose layers learn by delta-rule steps
    (DeltaTTT summary, paperlayer.ai, §4.1 "Layerwise memory optimization" and
    §4.1 on the Pre schedule; Appendix A, chunkwise scan).

    The first layer A [dv, dk] learns keys -> values; the second layer
    B [dv, dv] learns intermediate representation -> value, so that it can
    correct the first layer's prediction.  In the Pre schedule the
    intermediate representation of token t is formed from the first layer's
    state before token t's write, so the two writes of a token are independent.
    Readings (the summary prints no formulas): the nonlinearity is SiLU (the
    two-layer SiLU memories of its Appendix B); the second layer's write key is
    the unit-normalised SiLU of the first layer's prediction, like the unit keys
    of the first layer; the query goes through the first layer after its write
    (readout after write, as in the delta rule) and the same SiLU and
    normalisation; each layer has its own step size and decay of the given
    variant ("deltanet" or "gdn").  The structure (two delta-rule layers, the
    Pre write key, two scans) is pinned; the choice of SiLU and of the unit
    normalisation of h and z is parity unpinned: nothing on the pages fixes
    them.  Per token, float64:

        A' = A a1_t;       r = A' k_t;     A = A' + beta1_t (v_t - r) k_t^T
        h  = unit(silu(r));                z = unit(silu(A q_t))
        B' = B a2_t;       s = B' h;       B = B' + beta2_t (v_t - s) h^T
        o_t = B z

    q, k [B, T, H, dk]; v [B, T, H, dv]; beta1, beta2 [B, T, H]; g1, g2 [B, T, H]
    for "gdn" (None for "deltanet"); A0 [B, H, dv, dk] and B0 [B, H, dv, dv] or
    None (zero).  Returns o [B, T, H, dv], A_T, B_T; with ``internals`` also the
    per-token h and z [B, T, H, dv].
    """
    if variant not in ("deltanet", "gdn"):
        raise ValueError("DeltaTTT-pre takes the deltanet or gdn form")
    B, T, H, dv = np.shape(v)
    dk = np.shape(q)[3]
    q, k, v = (_to_heads(x) for x in (q, k, v))
    b1, b2 = _to_heads(beta1), _to_heads(beta2)
    a1 = _to_heads(_decay(variant, g1, (B, T, H), dk))
    a2 = _to_heads(_decay(variant, g2, (B, T, H), dv))
    A = (np.zeros((B * H, dv, dk)) if A0 is None
         else np.asarray(A0, dtype=np.float64).reshape(B * H, dv, dk).copy())
    Bm = (np.zeros((B * H, dv, dv)) if B0 is None
          else np.asarray(B0, dtype=np.float64).reshape(B * H, dv, dv).copy())
    o = np.empty((B * H, T, dv))
    hs = np.empty((B * H, T, dv))
    zs = np.empty((B * H, T, dv))
    for t in range(T):
        kt, qt, vt = k[:, t], q[:, t], v[:, t]
        Ap = A * a1[:, t, None, :]
        r = (Ap @ kt[:, :, None])[:, :, 0]
        A = Ap + b1[:, t, None, None] * (vt - r)[:, :, None] * kt[:, None, :]
        h = _unit_rows(_silu(r))
        z = _unit_rows(_silu((A @ qt[:, :, None])[:, :, 0]))
        Bp = Bm * a2[:, t, None, :]
        s = (Bp @ h[:, :, None])[:, :, 0]
        Bm = Bp + b2[:, t, None, None] * (vt - s)[:, :, None] * h[:, None, :]
        o[:, t] = (Bm @ z[:, :, None])[:, :, 0]
        hs[:, t], zs[:, t] = h, z
    back = lambda x: np.ascontiguousarray(np.moveaxis(x.reshape(B, H, T, -1), 1, 2))  # noqa: E731
    out = (back(o), A.reshape(B, H, dv, dk), Bm.reshape(B, H, dv, dv))
    if internals:
        out = out + (back(hs), back(zs))
    return out
