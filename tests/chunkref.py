"""Float64 CPU chunkwise reference: the chunk algebra the HIP prefill kernel uses.

Test helper only.  It is compared with the token-by-token oracle (exact up to
rounding) and, when a GPU parity case fails, against the kernel's output to
localise the fault.  It shares no code with the HIP path or the oracle.

The recurrence is affine in the preceding memory (DeltaTTT summary,
paperlayer.ai, §2 Background), so a chunk of C tokens acts on its incoming
state S in closed form.  With G the in-chunk cumulative log-decay (G_r =
g_1 + ... + g_r; per key channel for channel-wise decay), K^ = K ⊙ e^G,
Q^ = Q ⊙ e^G, K- = K ⊙ e^(G_C - G) and the C×C matrices (rows r, columns j)

    A_k[r, j] = Σ_c k_rc k_jc e^(G_rc - G_jc)      (j < r)
    M_k[r, j] = Σ_c q_rc k_jc e^(G_rc - G_jc)      (j ≤ r)

single step size (DeltaNet, Gated DeltaNet, KDA):

    T = (I + diag(β) A_k)^-1
    V~ = T diag(β) (V - K^ S^T)               row j = β_j (v_j - S'_j k_j)
    O  = Q^ S^T + M_k V~
    S^T <- Diag(e^G_C) S^T + K-^T V~

split erase/write gates (Gated DeltaNet-2, erase b on the key side, write w on
the value side, X = w ⊙ V, E = b ⊙ K):

    A_e[r, j] = Σ_c k_rc e_jc e^(G_rc - G_jc)  (j < r);  M_e likewise with q (j ≤ r)
    T = (I + A_e)^-1
    Y = T (K^ S^T + A_k X)                    row j = S'_j k_j, the erase read
    O = Q^ S^T + M_k X - M_e Y
    S^T <- Diag(e^G_C) S^T + K-^T X - E-^T Y    (E- = E ⊙ e^(G_C - G))

step size per key channel (FG^2-GDN, E = beta ⊙ K): the split form with the
write along E instead of K and no write gate, i.e. X = V, A_k -> A_e,
M_k -> M_e and K- -> E-:

    Y = T (K^ S^T + A_e V)
    O = Q^ S^T + M_e (V - Y)
    S^T <- Diag(e^G_C) S^T + E-^T (V - Y)

These follow the chunkwise WY description of the Gated DeltaNet-2 abstract
(thelatestinai.com/papers/2607.07953), derived here from the token update.
"""
from __future__ import annotations

import numpy as np


def _heads(x):
    if x is None:
        return None
    x = np.asarray(x, dtype=np.float64)
    B, T, H = x.shape[:3]
    return np.moveaxis(x, 2, 1).reshape((B * H, T) + x.shape[3:])


def chunk_fwd(variant, q, k, v, beta=None, wgate=None, g=None, S0=None, chunk=64):
    """Chunkwise forward in float64; same argument layout as the oracle's delta_fwd."""
    q64 = np.asarray(q, dtype=np.float64)
    B, T, H, dk = q64.shape
    dv = np.shape(v)[3]
    N = B * H
    Q, K, V = _heads(q), _heads(k), _heads(v)
    if variant == "deltanet":
        G_tok = np.zeros((N, T, dk))
    elif variant == "gdn":
        G_tok = np.broadcast_to(_heads(g)[..., None], (N, T, dk))
    else:
        G_tok = _heads(g)
    split = variant in ("gdn2", "fg2")
    keywrite = variant == "fg2"
    if split:
        E_all = _heads(beta)
        W_all = None if keywrite else _heads(wgate)
    else:
        Bt = _heads(beta)
    S_T = np.zeros((N, dk, dv)) if S0 is None else np.swapaxes(
        np.asarray(S0, dtype=np.float64).reshape(N, dv, dk), 1, 2).copy()
    O = np.zeros((N, T, dv))
    for n0 in range(0, T, chunk):
        n1 = min(n0 + chunk, T)
        C = n1 - n0
        Kc, Qc, Vc = K[:, n0:n1], Q[:, n0:n1], V[:, n0:n1]
        G = np.cumsum(G_tok[:, n0:n1], axis=1)                     # [N, C, dk]
        GC = G[:, -1:, :]                                           # [N, 1, dk]
        lower = np.tril(np.ones((C, C)), -1)
        lower0 = np.tril(np.ones((C, C)))
        # entries above the diagonal are never used and may overflow: mask them
        with np.errstate(over="ignore"):
            diff = np.exp(G[:, :, None, :] - G[:, None, :, :])      # [N, r, j, dk]
        diff = np.where(lower0[None, :, :, None] > 0, diff, 0.0)
        Ak = np.einsum("nrc,njc,nrjc->nrj", Kc, Kc, diff) * lower
        Mk = np.einsum("nrc,njc,nrjc->nrj", Qc, Kc, diff) * lower0
        Kh, Qh, Kb = Kc * np.exp(G), Qc * np.exp(G), Kc * np.exp(GC - G)
        XS = Kh @ S_T                                               # [N, C, dv]
        eye = np.eye(C)
        if not split:
            bt = Bt[:, n0:n1]
            Tm = np.linalg.inv(eye + bt[:, :, None] * Ak)
            Vt = Tm @ (bt[:, :, None] * (Vc - XS))
            O[:, n0:n1] = Qh @ S_T + Mk @ Vt
            S_T = np.exp(GC[:, 0, :])[:, :, None] * S_T + np.swapaxes(Kb, 1, 2) @ Vt
        else:
            Ec = E_all[:, n0:n1] * Kc
            Ae = np.einsum("nrc,njc,nrjc->nrj", Kc, Ec, diff) * lower
            Me = np.einsum("nrc,njc,nrjc->nrj", Qc, Ec, diff) * lower0
            Eb = Ec * np.exp(GC - G)
            if keywrite:
                X, Ak, Mk, Kb = Vc, Ae, Me, Eb
            else:
                X = W_all[:, n0:n1] * Vc
            Tm = np.linalg.inv(eye + Ae)
            Y = Tm @ (XS + Ak @ X)
            O[:, n0:n1] = Qh @ S_T + Mk @ X - Me @ Y
            S_T = (np.exp(GC[:, 0, :])[:, :, None] * S_T + np.swapaxes(Kb, 1, 2) @ X
                   - np.swapaxes(Eb, 1, 2) @ Y)
    o = np.moveaxis(O.reshape(B, H, T, dv), 1, 2)
    return np.ascontiguousarray(o), np.swapaxes(S_T, 1, 2).reshape(B, H, dv, dk)
