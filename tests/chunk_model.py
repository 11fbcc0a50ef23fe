"""fp64 model of the chunkwise WY form (test-only design check).

It restates the chunk algebra that the HIP prefill follows, in plain numpy,
so that the algebra can be checked against the sequential oracle without a
GPU. Shares no code with the kernels or the oracle.

Within a chunk of n tokens starting from state S0 (d_k x d_v), with
g_r = sum_{s<=r} log alpha_s (per key channel) and u_r = w_r * v_r, the
recurrence unrolls to (snilld.dk, "Hvad betyder det for træning og
inferens": chunkwise WY form, cumulative decay folded into the rank-one erase
factors):
    A_rs   = sum_c b_rc k_rc k_sc exp(g_rc - g_sc)       (s < r)
    Delta  = (I + A)^{-1} (U - E S0),  E_r = b_r * k_r * exp(g_r)
    P_rs   = sum_c q_rc k_sc exp(g_rc - g_sc)            (s <= r)
    O      = Q+ S0 + P Delta,           Q+_r = q_r * exp(g_r)
    S_n    = Diag(exp(g_n)) S0 + Khat^T Delta,  Khat_s = k_s * exp(g_n - g_s)
`rnd` (optional) rounds every matrix-product operand, to model reduced
precision operands.
"""
import numpy as np


def chunk_forward(q, k, v, la, b, w, S0=None, cu_seqlens=None, C=64, rnd=None):
    r = (lambda x: x) if rnd is None else rnd
    T, H, dk = q.shape
    dv = v.shape[-1]
    cu = np.asarray([0, T] if cu_seqlens is None else cu_seqlens)
    N = len(cu) - 1
    o = np.zeros((T, H, dv))
    ST = np.zeros((N, H, dk, dv))
    for i in range(N):
        for h in range(H):
            S = np.zeros((dk, dv)) if S0 is None else S0[i, h].astype(np.float64).copy()
            for c0 in range(cu[i], cu[i + 1], C):
                sl = slice(c0, min(c0 + C, cu[i + 1]))
                n = sl.stop - sl.start
                g = np.cumsum(la[sl, h], axis=0)
                diff = g[:, None, :] - g[None, :, :]                     # [r, s, c]
                causal = np.tril(np.ones((n, n), bool))
                dec = np.where(causal[:, :, None], np.exp(np.where(causal[:, :, None], diff, 0.0)), 0.0)
                A = np.einsum('rc,rsc,sc->rs', b[sl, h] * k[sl, h], dec, k[sl, h]) * (1 - np.eye(n))
                P = np.einsum('rc,rsc,sc->rs', q[sl, h], dec, k[sl, h])
                Tinv = np.linalg.solve(np.eye(n) + A, np.eye(n))
                E = b[sl, h] * k[sl, h] * np.exp(g)
                U = w[sl, h] * v[sl, h]
                Delta = r(Tinv) @ r(U) - r(r(Tinv) @ r(E)) @ r(S)
                o[sl, h] = r(q[sl, h] * np.exp(g)) @ r(S) + r(P) @ r(Delta)
                Khat = k[sl, h] * np.exp(g[-1][None, :] - g)
                S = np.exp(g[-1])[:, None] * S + r(Khat).T @ r(Delta)
            ST[i, h] = S
    return o, ST


def chunk_backward(q, k, v, la, b, w, dO, S0=None, dST=None, cu_seqlens=None, C=64):
    """Gradients of sum(dO * o) + sum(dST * S_T) through the chunk form above.

    Per chunk, with S_c its start state and G the gradient at its end state:
        dDelta = P^T dO + Khat G,       dX = T^T dDelta      (X = U - E S_c)
        dS_c   = Q+^T dO + Diag(e^{g_n}) G - E^T dX
        dU = dX,   dA = -strict_tril(dX Delta^T),   dP = tril(dO Delta^T)
        dQ+ = dO S_c^T + dP K-,  dK- = dP^T Q+ + dA^T E,  dE = -dX S_c^T + dA K-
        dKhat = Delta G^T,       dgamma = diag(G S_c^T)
    (K-_s = k_s e^{-g_s}), then through the decay factors to q, k, b and the
    cumulative g (reverse cumulative sum within the chunk gives d log alpha).
    Products with e^{-g} are formed with pairwise exponents g_r - g_s <= 0.
    """
    T, H, dk = q.shape
    dv = v.shape[-1]
    cu = np.asarray([0, T] if cu_seqlens is None else cu_seqlens)
    N = len(cu) - 1
    g_ = {n: np.zeros(x.shape) for n, x in (('q', q), ('k', k), ('v', v), ('log_alpha', la), ('b', b), ('w', w))}
    g_['S0'] = np.zeros((N, H, dk, dv))
    for i in range(N):
        for h in range(H):
            S = np.zeros((dk, dv)) if S0 is None else S0[i, h].astype(np.float64).copy()
            chunks = list(range(cu[i], cu[i + 1], C))
            starts = []
            for c0 in chunks:                       # forward: chunk start states
                starts.append(S.copy())
                sl = slice(c0, min(c0 + C, cu[i + 1]))
                n = sl.stop - sl.start
                gg = np.cumsum(la[sl, h], axis=0)
                causal = np.tril(np.ones((n, n), bool))
                diff = gg[:, None, :] - gg[None, :, :]
                dec = np.where(causal[:, :, None], np.exp(np.where(causal[:, :, None], diff, 0.0)), 0.0)
                A = np.einsum('rc,rsc,sc->rs', b[sl, h] * k[sl, h], dec, k[sl, h]) * (1 - np.eye(n))
                Tinv = np.linalg.solve(np.eye(n) + A, np.eye(n))
                E = b[sl, h] * k[sl, h] * np.exp(gg)
                Delta = Tinv @ (w[sl, h] * v[sl, h] - E @ S)
                S = np.exp(gg[-1])[:, None] * S + (k[sl, h] * np.exp(gg[-1][None, :] - gg)).T @ Delta
            G = np.zeros((dk, dv)) if dST is None else dST[i, h].astype(np.float64).copy()
            for c0, Sc in reversed(list(zip(chunks, starts))):
                sl = slice(c0, min(c0 + C, cu[i + 1]))
                n = sl.stop - sl.start
                qq, kk, bb, vv, ww, dOc = q[sl, h], k[sl, h], b[sl, h], v[sl, h], w[sl, h], dO[sl, h]
                gg = np.cumsum(la[sl, h], axis=0)
                causal = np.tril(np.ones((n, n), bool))
                diff = gg[:, None, :] - gg[None, :, :]
                dec = np.where(causal[:, :, None], np.exp(np.where(causal[:, :, None], diff, 0.0)), 0.0)
                A = np.einsum('rc,rsc,sc->rs', bb * kk, dec, kk) * (1 - np.eye(n))
                P = np.einsum('rc,rsc,sc->rs', qq, dec, kk)
                Tinv = np.linalg.solve(np.eye(n) + A, np.eye(n))
                E = bb * kk * np.exp(gg)
                U = ww * vv
                X = U - E @ Sc
                Delta = Tinv @ X
                Khat = kk * np.exp(gg[-1][None, :] - gg)
                gam = np.exp(gg[-1])
                dDelta = P.T @ dOc + Khat @ G
                dX = Tinv.T @ dDelta
                dA = -(dX @ Delta.T) * np.tril(np.ones((n, n)), -1)
                dP = (dOc @ Delta.T) * np.tril(np.ones((n, n)))
                # physical gradients, pairwise exponents where e^{-g} appears
                dq = (dOc @ Sc.T) * np.exp(gg) + np.einsum('rs,rsc,sc->rc', dP, dec, kk)
                dk_km = np.einsum('rs,rsc,rc->sc', dP, dec, qq) + np.einsum('rs,rsc,rc->sc', dA, dec, bb * kk)
                dEe = -(dX @ Sc.T) * np.exp(gg) + np.einsum('rs,rsc,sc->rc', dA, dec, kk)   # dE * e^g
                dk_kh = (Delta @ G.T) * np.exp(gg[-1][None, :] - gg)
                dgam = np.sum(G * Sc, axis=1)
                g_['q'][sl, h] = dq
                g_['k'][sl, h] = dk_km + dk_kh + dEe * bb
                g_['b'][sl, h] = dEe * kk
                g_['v'][sl, h] = dX * ww
                g_['w'][sl, h] = dX * vv
                dG = dq * qq - dk_km * kk - dk_kh * kk + dEe * bb * kk
                dG[-1] += np.sum(dk_kh * kk, axis=0) + dgam * gam
                g_['log_alpha'][sl, h] = np.cumsum(dG[::-1], axis=0)[::-1]
                G = (qq * np.exp(gg)).T @ dOc + gam[:, None] * G - E.T @ dX
            g_['S0'][i, h] = G
    return g_
