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
