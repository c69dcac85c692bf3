"""fp64 CPU model of the chunkwise backward that the HIP kernels implement
(single step size: DeltaNet, GDN, KDA; split gates: Gated DeltaNet-2 below).  Test infrastructure only: it shares no
code with the oracle or the kernels and is compared with the oracle's token-level
reverse mode in test_chunkref_bwd.py.

Per chunk of C rows with incoming state S [dv, dk] (Gated DeltaNet-2 abstract:
chunkwise WY form with the decay absorbed into the key factors; here every
factor that could overflow is taken pairwise, e^{G_r - G_j} with j <= r):

    E[r, j]  = exp(G_r - G_j) per key channel, j <= r
    Abar     = StrictTril(sum_c k_r k_j E),  A = diag(beta) Abar,  T = (I + A)^-1
    Khat     = k e^G,  Qhat = q e^G,  Kbar = k e^{G_C - G},  gamma = e^{G_C}
    X = beta Khat,  Y = beta v,  W = T X,  U = T Y
    Mq       = Tril0(sum_c q_r k_j E)
    Vt       = U - W S^T
    O        = Qhat S^T + Mq Vt
    S_next   = S Diag(gamma) + Vt^T Kbar

The backward runs the state chain in reverse (dS carried from chunk to chunk)
and then, per chunk, the gradients of every factor above.
"""
import numpy as np


def _chunk_factors(q, k, v, beta, g):
    C = q.shape[0]
    G = np.cumsum(g, axis=0)                           # [C, dk]
    diff = G[:, None, :] - G[None, :, :]               # G_r - G_j
    low = np.tril(np.ones((C, C), dtype=bool))
    E = np.where(low[:, :, None], np.exp(np.where(low[:, :, None], diff, 0.0)), 0.0)
    Abar = np.einsum("rc,jc,rjc->rj", k, k, E) * np.tril(np.ones((C, C)), -1)
    A = beta[:, None] * Abar
    T = np.linalg.inv(np.eye(C) + A)
    eG = np.exp(G)
    Khat, Qhat = k * eG, q * eG
    Kbar = k * np.exp(G[-1][None, :] - G)
    gamma = np.exp(G[-1])
    X, Y = beta[:, None] * Khat, beta[:, None] * v
    Mq = np.einsum("rc,jc,rjc->rj", q, k, E) * low
    return dict(G=G, E=E, Abar=Abar, T=T, eG=eG, Khat=Khat, Qhat=Qhat, Kbar=Kbar, gamma=gamma,
                X=X, Y=Y, W=T @ X, U=T @ Y, Mq=Mq)


def chunk_forward(q, k, v, beta, g, S0, C=64):
    """One head: q, k [T, dk], v [T, dv], beta [T], g [T, dk] (zeros for DeltaNet,
    a broadcast scalar for GDN), S0 [dv, dk].  Returns o, the final state, and the
    per-chunk factors and incoming states the backward needs."""
    T = q.shape[0]
    S = np.array(S0, dtype=np.float64)
    o = np.zeros((T, v.shape[1]))
    saved = []
    for t0 in range(0, T, C):
        sl = slice(t0, min(T, t0 + C))
        f = _chunk_factors(q[sl], k[sl], v[sl], beta[sl], g[sl])
        Vt = f["U"] - f["W"] @ S.T
        o[sl] = f["Qhat"] @ S.T + f["Mq"] @ Vt
        saved.append((sl, f, S, Vt))
        S = S * f["gamma"][None, :] + Vt.T @ f["Kbar"]
    return o, S, saved


def chunk_backward(q, k, v, beta, g, S0, dO, dST, C=64):
    """Gradients for one head (same layout as chunk_forward); dST may be None.
    Returns dq, dk, dv, dbeta, dg [T, dk] (per channel; sum over channels for GDN)
    and dS0."""
    _, _, saved = chunk_forward(q, k, v, beta, g, S0, C)
    T, dk = q.shape
    dq, dkk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    dbeta, dg = np.zeros(T), np.zeros((T, dk))
    dSn = np.zeros((v.shape[1], dk)) if dST is None else np.array(dST, dtype=np.float64)
    for sl, f, S, Vt in reversed(saved):
        qc, kc, vc, bc, dOc = q[sl], k[sl], v[sl], beta[sl], dO[sl]
        E, Tm = f["E"], f["T"]
        # reverse state chain
        dVt = f["Mq"].T @ dOc + f["Kbar"] @ dSn.T
        dS = dSn * f["gamma"][None, :] + dOc.T @ f["Qhat"] - dVt.T @ f["W"]
        # per-chunk gradients
        dMq = np.tril(dOc @ Vt.T)
        dQhat = dOc @ S
        dKbar = Vt @ dSn
        dW, dU = -dVt @ S, dVt
        dT = dW @ f["X"].T + dU @ f["Y"].T
        dX, dY = Tm.T @ dW, Tm.T @ dU
        dA = np.tril(-Tm.T @ dT @ Tm.T, -1)
        dv[sl] = bc[:, None] * dY
        dbeta[sl] = (np.sum(dY * vc, axis=1) + np.sum(dX * f["Khat"], axis=1)
                     + np.sum(dA * f["Abar"], axis=1))
        dAbar = bc[:, None] * dA
        dKhat = bc[:, None] * dX
        # pairwise products: P1[r, j, c] = dMq[r, j] q_rc k_jc E, P2 likewise with dAbar, k_r
        P1 = dMq[:, :, None] * qc[:, None, :] * kc[None, :, :] * E
        P2 = dAbar[:, :, None] * kc[:, None, :] * kc[None, :, :] * E
        dqc = dQhat * f["eG"] + np.einsum("rj,jc,rjc->rc", dMq, kc, E)
        dkc = (np.einsum("rj,rc,rjc->jc", dMq, qc, E) + np.einsum("rj,jc,rjc->rc", dAbar, kc, E)
               + np.einsum("rj,rc,rjc->jc", dAbar, kc, E)
               + dKhat * f["eG"] + dKbar * np.exp(f["G"][-1][None, :] - f["G"]))
        dG = (P1.sum(axis=1) - P1.sum(axis=0) + P2.sum(axis=1) - P2.sum(axis=0)
              + dKhat * f["Khat"] + dQhat * f["Qhat"] - dKbar * f["Kbar"])
        dG[-1] += np.sum(dKbar * f["Kbar"], axis=0) + f["gamma"] * np.sum(S * dSn, axis=0)
        dq[sl], dkk[sl] = dqc, dkc
        dg[sl] = np.cumsum(dG[::-1], axis=0)[::-1]
        dSn = dS
    return dq, dkk, dv, dbeta, dg, dSn


# ------------------------------------------------------------- split gates
# Gated DeltaNet-2 (erase gate b on the key side, write gate w on the value
# side), pairwise like the above:
#     Ae = StrictTril(sum_c k_r (b k)_j E),  Ak = StrictTril(sum_c k_r k_j E),
#     T = (I + Ae)^-1,  X = w v,  Z = Ak X,  W = T Khat,  Ut = T Z
#     Me = Tril0(sum_c q_r (b k)_j E),  Mk = Tril0(sum_c q_r k_j E)
#     Ebar = (b k) e^{G_C - G}
#     Y = W S^T + Ut,  O = Qhat S^T - Me Y + Mk X,
#     S_next = S Diag(gamma) - Y^T Ebar + X^T Kbar


def _chunk_factors2(q, k, v, b, w, g):
    C = q.shape[0]
    G = np.cumsum(g, axis=0)
    diff = G[:, None, :] - G[None, :, :]
    low = np.tril(np.ones((C, C), dtype=bool))
    E = np.where(low[:, :, None], np.exp(np.where(low[:, :, None], diff, 0.0)), 0.0)
    bk = b * k
    strict = np.tril(np.ones((C, C)), -1)
    Ae = np.einsum("rc,jc,rjc->rj", k, bk, E) * strict
    Ak = np.einsum("rc,jc,rjc->rj", k, k, E) * strict
    T = np.linalg.inv(np.eye(C) + Ae)
    eG = np.exp(G)
    ebar = np.exp(G[-1][None, :] - G)
    X = w * v
    Z = Ak @ X
    Khat = k * eG
    return dict(G=G, E=E, bk=bk, Ae=Ae, Ak=Ak, T=T, eG=eG, ebar=ebar, X=X, Z=Z, Khat=Khat,
                Qhat=q * eG, Kbar=k * ebar, Ebar=bk * ebar, gamma=np.exp(G[-1]), W=T @ Khat,
                Ut=T @ Z, Me=np.einsum("rc,jc,rjc->rj", q, bk, E) * low,
                Mk=np.einsum("rc,jc,rjc->rj", q, k, E) * low)


def chunk_forward2(q, k, v, b, w, g, S0, C=64):
    T = q.shape[0]
    S = np.array(S0, dtype=np.float64)
    o = np.zeros((T, v.shape[1]))
    saved = []
    for t0 in range(0, T, C):
        sl = slice(t0, min(T, t0 + C))
        f = _chunk_factors2(q[sl], k[sl], v[sl], b[sl], w[sl], g[sl])
        Y = f["W"] @ S.T + f["Ut"]
        o[sl] = f["Qhat"] @ S.T - f["Me"] @ Y + f["Mk"] @ f["X"]
        saved.append((sl, f, S, Y))
        S = S * f["gamma"][None, :] - Y.T @ f["Ebar"] + f["X"].T @ f["Kbar"]
    return o, S, saved


def chunk_backward2(q, k, v, b, w, g, S0, dO, dST, C=64):
    """Gradients for one head of the split-gate form: dq, dk, dv, db, dw, dg
    (per channel) and dS0."""
    _, _, saved = chunk_forward2(q, k, v, b, w, g, S0, C)
    T, dk = q.shape
    out = {n: np.zeros_like(a) for n, a in (("dq", q), ("dk", k), ("dv", v), ("db", b), ("dw", w))}
    dgs = np.zeros((T, dk))
    dSn = np.zeros((v.shape[1], dk)) if dST is None else np.array(dST, dtype=np.float64)
    for sl, f, S, Y in reversed(saved):
        qc, kc, vc, bc, wc, dOc = q[sl], k[sl], v[sl], b[sl], w[sl], dO[sl]
        E, Tm, X = f["E"], f["T"], f["X"]
        # reverse state chain
        dY = -f["Me"].T @ dOc - f["Ebar"] @ dSn.T
        dS = dSn * f["gamma"][None, :] + dOc.T @ f["Qhat"] + dY.T @ f["W"]
        # per-chunk gradients
        dMe = -np.tril(dOc @ Y.T)
        dMk = np.tril(dOc @ X.T)
        dQhat = dOc @ S
        dW = dY @ S
        dUt = dY
        dEbar = -Y @ dSn
        dKbar = X @ dSn
        dZ = Tm.T @ dUt
        dT = dW @ f["Khat"].T + dUt @ f["Z"].T
        dAe = np.tril(-Tm.T @ dT @ Tm.T, -1)
        dAk = np.tril(dZ @ X.T, -1)
        dX = f["Mk"].T @ dOc + f["Kbar"] @ dSn.T + f["Ak"].T @ dZ
        dKhat = Tm.T @ dW
        out["dv"][sl] = wc * dX
        out["dw"][sl] = vc * dX
        # pairwise sums, per channel: "row" terms index r (left factor), "col" terms j
        def row(M, R):   # sum_j M[r, j] R_j E[r, j]
            return np.einsum("rj,jc,rjc->rc", M, R, E)

        def col(M, L):   # sum_r M[r, j] L_r E[r, j]
            return np.einsum("rj,rc,rjc->jc", M, L, E)

        dq_ = dQhat * f["eG"] + row(dMe, f["bk"]) + row(dMk, kc)
        dk_ = (row(dAe, f["bk"]) + row(dAk, kc) + col(dAk, kc) + col(dMk, qc)
               + dKhat * f["eG"] + dKbar * f["ebar"])
        dbk = col(dAe, kc) + col(dMe, qc) + dEbar * f["ebar"]
        dG = (qc * row(dMe, f["bk"]) - f["bk"] * col(dMe, qc) + qc * row(dMk, kc) - kc * col(dMk, qc)
              + kc * row(dAe, f["bk"]) - f["bk"] * col(dAe, kc) + kc * row(dAk, kc) - kc * col(dAk, kc)
              + dKhat * f["Khat"] + dQhat * f["Qhat"] - dKbar * f["Kbar"] - dEbar * f["Ebar"])
        dG[-1] += (np.sum(dKbar * f["Kbar"], axis=0) + np.sum(dEbar * f["Ebar"], axis=0)
                   + f["gamma"] * np.sum(S * dSn, axis=0))
        out["dq"][sl] = dq_
        out["dk"][sl] = dk_ + dbk * bc
        out["db"][sl] = dbk * kc
        dgs[sl] = np.cumsum(dG[::-1], axis=0)[::-1]
        dSn = dS
    out["dg"] = dgs
    out["dS0"] = dSn
    return out
