"""Pins for the oracle: checks against what the pages and the mathematics fix.

Each pin takes a forward callable with the oracle's signature,
``fwd(q, k, v, log_alpha, b, w, S0=None, cu_seqlens=None, B=None) -> (o, S_T)``
on token tensors ``[tokens, H, d]``, so the same pins can run against planted
mistakes (see test_oracle_mutants.py). None of them re-types the oracle's
rank-one loop: each compares it with a different formulation (a dense matrix
product, a textbook rule the pages reduce to, a closed form, an invariant, a
hand-worked example).

Sources (page title, section):
  GDR2   snilld.dk, "Hvad Gated DeltaNet-2 ændrer": the update equation with
         channel-wise decay before the edit, and its collapse to KDA (both
         gates the same scalar) and to Gated DeltaNet (alpha scalar too).
  P2EQ   aifetchly, "Gated DeltaNet-2 Guide", "1. Decoupled Erase and Write
         Gates": the alpha-free update written for the transposed state.
  P2LOOP aifetchly, "End-to-End PyTorch Implementation": readout after the
         update, zero initial state, (output, final_state) returned.
  DELTA  aifetchly, "The Classical Delta Rule and Memory Saturation": the
         Widrow-Hoff update S_t = S_{t-1} - beta (S_{t-1} k - v) k^T.
  HEBB   aifetchly, "The Associative Memory Dilemma" diagram, item 1 (linear
         attention S_t = S_{t-1} + v k^T) and "The Four Modes", mode 3.
  MODES  aifetchly, "The Four Modes of Expressive Memory Editing".
  SPEC   aifetchly, "2. Normalization and Short Convolutions" (spectrum of
         the erase factor).
"""
from __future__ import annotations

import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), 'golden')


def rand_inputs(rng, T, H, dk, dv, unit_k=True, s0=0.3):
    q = rng.standard_normal((T, H, dk))
    k = rng.standard_normal((T, H, dk))
    if unit_k:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H, dv))
    la = -np.logaddexp(0, rng.standard_normal((T, H, dk)) - 2.0)
    b = 1 / (1 + np.exp(-rng.standard_normal((T, H, dk))))
    w = 1 / (1 + np.exp(-rng.standard_normal((T, H, dv))))
    S0 = s0 * rng.standard_normal((1, H, dk, dv))
    return q, k, v, la, b, w, S0


# ---------------------------------------------------------------- helpers

def dense_recurrence(q, k, v, la, b, w, S0):
    """GDR2 as printed: the full matrix (I - k (b*k)^T) Diag(alpha) times S."""
    T, H, dk = q.shape
    dv = v.shape[-1]
    o = np.zeros((T, H, dv))
    ST = np.zeros((1, H, dk, dv))
    for h in range(H):
        S = S0[0, h].copy() if S0 is not None else np.zeros((dk, dv))
        for t in range(T):
            M = (np.eye(dk) - np.outer(k[t, h], b[t, h] * k[t, h])) @ np.diag(np.exp(la[t, h]))
            S = M @ S + np.outer(k[t, h], w[t, h] * v[t, h])
            o[t, h] = S.T @ q[t, h]
        ST[0, h] = S
    return o, ST


def load_golden(name):
    rows = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split('#', 1)[0].strip()
            if not line:
                continue
            parts = line.split()
            rows[(parts[0], int(parts[1]))] = np.array([float(x) for x in parts[2:]])
    return rows


def close(a, b, tol, what):
    err = np.max(np.abs(np.asarray(a) - np.asarray(b))) if np.size(a) else 0.0
    assert err <= tol, f'{what}: max abs diff {err:.3e} > {tol:.1e}'


# ---------------------------------------------------------------- pins

def pin_dense_product(fwd):
    """Brute force: the printed matrix product, random alpha, b, w, S0 != 0."""
    rng = np.random.default_rng(11)
    for dk, dv, T in ((5, 3, 40), (16, 12, 64), (4, 7, 33)):
        q, k, v, la, b, w, S0 = rand_inputs(rng, T, 2, dk, dv)
        k = k * rng.uniform(0.6, 1.2, size=(T, 2, 1))   # keys off the unit sphere too
        o, ST = fwd(q, k, v, la, b, w, S0)
        o_ref, ST_ref = dense_recurrence(q, k, v, la, b, w, S0)
        close(o, o_ref, 1e-11, 'o vs dense product')
        close(ST, ST_ref, 1e-11, 'S_T vs dense product')


def pin_hand_worked(fwd):
    """The three-token example in tests/golden/hand_worked_2x2.txt (GDR2)."""
    g = load_golden('hand_worked_2x2.txt')
    T = 3
    arr = {n: np.stack([g[(n, t)] for t in range(1, T + 1)])[:, None, :]
           for n in ('q', 'k', 'v', 'alpha', 'b', 'w')}
    o, ST = fwd(arr['q'], arr['k'], arr['v'], np.log(arr['alpha']), arr['b'], arr['w'], None)
    o_ref = np.stack([g[('o', t)] for t in range(1, T + 1)])[:, None, :]
    ST_ref = np.stack([g[('ST', 0)], g[('ST', 1)]])[None, None]
    close(o, o_ref, 1e-12, 'hand-worked o')
    close(ST, ST_ref, 1e-12, 'hand-worked S_T')


def pin_alpha_free_transposed(fwd):
    """P2EQ/P2LOOP with alpha = 1: S' = S' (I - (b*k) k^T) + (w*v) k^T, y = S' q,
    where S' (d_v x d_k) is the transpose of the state."""
    rng = np.random.default_rng(12)
    T, H, dk, dv = 50, 2, 8, 6
    q, k, v, la, b, w, S0 = rand_inputs(rng, T, H, dk, dv)
    la = np.zeros_like(la)
    o, ST = fwd(q, k, v, la, b, w, S0)
    for h in range(H):
        Sp = S0[0, h].T.copy()
        for t in range(T):
            Sp = Sp @ (np.eye(dk) - np.outer(b[t, h] * k[t, h], k[t, h])) + np.outer(w[t, h] * v[t, h], k[t, h])
            close(o[t, h], Sp @ q[t, h], 1e-12, 'p2 readout')
        close(ST[0, h], Sp.T, 1e-12, 'p2 final state')


def pin_kda_collapse(fwd):
    """GDR2 with b = w = beta (scalar per token): KDA's S = (I - beta k k^T) Diag(alpha) S + beta k v^T."""
    rng = np.random.default_rng(13)
    T, H, dk, dv = 60, 2, 8, 5
    q, k, v, la, b, w, S0 = rand_inputs(rng, T, H, dk, dv)
    beta = rng.uniform(0.05, 0.95, size=(T, H))
    b = np.repeat(beta[:, :, None], dk, axis=2)
    w = np.repeat(beta[:, :, None], dv, axis=2)
    o, ST = fwd(q, k, v, la, b, w, S0)
    for h in range(H):
        S = S0[0, h].copy()
        for t in range(T):
            bt, kt = beta[t, h], k[t, h]
            S = (np.eye(dk) - bt * np.outer(kt, kt)) @ np.diag(np.exp(la[t, h])) @ S + bt * np.outer(kt, v[t, h])
            close(o[t, h], S.T @ q[t, h], 1e-12, 'KDA readout')
        close(ST[0, h], S, 1e-12, 'KDA state')


def pin_gdn_collapse(fwd):
    """GDR2 with scalar beta and scalar alpha = a: Gated DeltaNet, S = a (I - beta k k^T) S + beta k v^T."""
    rng = np.random.default_rng(14)
    T, H, dk, dv = 60, 2, 8, 5
    q, k, v, la, b, w, S0 = rand_inputs(rng, T, H, dk, dv)
    beta = rng.uniform(0.05, 0.95, size=(T, H))
    a = rng.uniform(0.8, 1.0, size=(T, H))
    b = np.repeat(beta[:, :, None], dk, axis=2)
    w = np.repeat(beta[:, :, None], dv, axis=2)
    la = np.repeat(np.log(a)[:, :, None], dk, axis=2)
    o, ST = fwd(q, k, v, la, b, w, S0)
    for h in range(H):
        S = S0[0, h].copy()
        for t in range(T):
            bt, kt = beta[t, h], k[t, h]
            S = a[t, h] * (S - bt * np.outer(kt, kt @ S)) + bt * np.outer(kt, v[t, h])
            close(o[t, h], S.T @ q[t, h], 1e-12, 'GDN readout')
        close(ST[0, h], S, 1e-12, 'GDN state')


def pin_textbook_delta_rule(fwd):
    """DELTA: alpha = 1, b = w = beta gives S' = S' - beta (S' k - v) k^T on the transposed state."""
    rng = np.random.default_rng(15)
    T, H, dk, dv = 60, 1, 6, 4
    q, k, v, la, b, w, S0 = rand_inputs(rng, T, H, dk, dv)
    beta = rng.uniform(0.1, 1.0, size=(T, H))
    b = np.repeat(beta[:, :, None], dk, axis=2)
    w = np.repeat(beta[:, :, None], dv, axis=2)
    la = np.zeros_like(la)
    o, ST = fwd(q, k, v, la, b, w, S0)
    Sp = S0[0, 0].T.copy()
    for t in range(T):
        Sp = Sp - beta[t, 0] * np.outer(Sp @ k[t, 0] - v[t, 0], k[t, 0])
        close(o[t, 0], Sp @ q[t, 0], 1e-12, 'delta-rule readout')
    close(ST[0, 0], Sp.T, 1e-12, 'delta-rule state')


def pin_linear_attention(fwd):
    """HEBB (b = 0, alpha = 1): causal linear attention in parallel form,
    O = Q S0 + tril(Q K^T) U and S_T = S0 + K^T U with U = w*v (two matmuls)."""
    rng = np.random.default_rng(16)
    T, H, dk, dv = 70, 2, 9, 7
    q, k, v, la, b, w, S0 = rand_inputs(rng, T, H, dk, dv, unit_k=False)
    b = np.zeros_like(b)
    la = np.zeros_like(la)   # with b = 0 any key norm is stable
    o, ST = fwd(q, k, v, la, b, w, S0)
    for h in range(H):
        Q, K, U = q[:, h], k[:, h], w[:, h] * v[:, h]
        close(o[:, h], Q @ S0[0, h] + np.tril(Q @ K.T) @ U, 1e-11, 'linear attention o')
        close(ST[0, h], S0[0, h] + K.T @ U, 1e-11, 'linear attention S_T')


def pin_decay_closed_form(fwd):
    """b = 0, any alpha: with G_t = sum_{s<=t} log alpha_s per channel,
    S_t = Diag(e^{G_t}) S0 + sum_{s<=t} Diag(e^{G_t - G_s}) k_s u_s^T (decay before the write)."""
    rng = np.random.default_rng(17)
    T, H, dk, dv = 50, 2, 6, 5
    q, k, v, la, b, w, S0 = rand_inputs(rng, T, H, dk, dv)
    b = np.zeros_like(b)
    o, ST = fwd(q, k, v, la, b, w, S0)
    for h in range(H):
        G = np.cumsum(la[:, h], axis=0)
        U = w[:, h] * v[:, h]
        for t in range(T):
            D = np.exp(G[t][None, :] - G[:t + 1])          # [s, c]
            S_t = np.exp(G[t])[:, None] * S0[0, h] + (k[:t + 1, h] * D).T @ U[:t + 1]
            close(o[t, h], S_t.T @ q[t, h], 1e-11, 'decay closed form o')
        close(ST[0, h], S_t, 1e-11, 'decay closed form S_T')


def pin_exact_retrieval(fwd):
    """b = 1, |k| = 1, any alpha: S_t^T k_t = w_t*v_t; with q = k the readout is w*v (MODES 1)."""
    rng = np.random.default_rng(18)
    T, H, dk, dv = 40, 2, 8, 6
    q, k, v, la, b, w, S0 = rand_inputs(rng, T, H, dk, dv)
    b = np.ones_like(b)
    o, ST = fwd(k, k, v, la, b, w, S0)
    close(o, w * v, 1e-12, 'exact retrieval')


def pin_pure_erase(fwd):
    """b = 1, w = 0, |k| = 1: the key is wiped, S_t^T k_t = 0 (MODES 2)."""
    rng = np.random.default_rng(19)
    T, H, dk, dv = 40, 2, 8, 6
    q, k, v, la, b, w, S0 = rand_inputs(rng, T, H, dk, dv)
    o, ST = fwd(k, k, v, la, np.ones_like(b), np.zeros_like(w), S0)
    close(o, np.zeros_like(o), 1e-12, 'pure erase')


def pin_preservation(fwd):
    """b = 0, w = 0, alpha = 1: the state passes unchanged (MODES 4)."""
    rng = np.random.default_rng(20)
    T, H, dk, dv = 30, 2, 7, 5
    q, k, v, la, b, w, S0 = rand_inputs(rng, T, H, dk, dv)
    o, ST = fwd(q, k, v, np.zeros_like(la), np.zeros_like(b), np.zeros_like(w), S0)
    close(ST, S0, 0.0, 'preserved state')
    close(o, np.einsum('thc,hcj->thj', q, S0[0]), 1e-12, 'preserved readout')


def pin_full_forget(fwd):
    """log alpha = -inf: the old state is gone, S_t = k_t (w_t*v_t)^T."""
    rng = np.random.default_rng(21)
    T, H, dk, dv = 20, 2, 6, 5
    q, k, v, la, b, w, S0 = rand_inputs(rng, T, H, dk, dv)
    o, ST = fwd(q, k, v, np.full_like(la, -np.inf), b, w, S0)
    u = w * v
    close(o, np.sum(k * q, axis=-1, keepdims=True) * u, 1e-12, 'full forget o')
    close(ST[0], np.einsum('hc,hj->hcj', k[-1], u[-1]), 1e-12, 'full forget S_T')


def pin_erase_spectrum(fwd):
    """SPEC: with alpha = 1, w = 0, one token maps S to (I - k (b*k)^T) S. Starting
    from S0 = I gives that matrix; its eigenvalues are 1 (d_k - 1 times) and
    1 - sum_c b_c k_c^2, inside [0, 1] for |k| = 1, although its operator norm
    can exceed 1 (the matrix is not normal)."""
    rng = np.random.default_rng(22)
    d = 8
    norms = []
    for _ in range(20):
        q, k, v, la, b, w, _ = rand_inputs(rng, 1, 1, d, d)
        o, ST = fwd(q, k, v, np.zeros_like(la), b, np.zeros_like(w), np.eye(d)[None, None])
        M = ST[0, 0]
        lam = np.sort(np.linalg.eigvals(M).real)
        expect = np.sort(np.r_[np.ones(d - 1), 1 - np.sum(b[0, 0] * k[0, 0] ** 2)])
        close(lam, expect, 1e-10, 'erase-factor eigenvalues')
        assert 0.0 <= lam.min() and lam.max() <= 1.0 + 1e-12
        close(M @ k[0, 0], k[0, 0] * (1 - np.sum(b[0, 0] * k[0, 0] ** 2)), 1e-12, 'k is the moving eigenvector')
        norms.append(np.linalg.norm(M, 2))
    assert max(norms) > 1.0


def pin_state_passing(fwd):
    """P2LOOP's (output, final_state): running [0, T) equals running [0, t) then [t, T) from its S_T."""
    rng = np.random.default_rng(23)
    T, H, dk, dv = 90, 2, 8, 6
    q, k, v, la, b, w, S0 = rand_inputs(rng, T, H, dk, dv)
    o, ST = fwd(q, k, v, la, b, w, S0)
    for t in (1, 37, 64):
        o1, S1 = fwd(q[:t], k[:t], v[:t], la[:t], b[:t], w[:t], S0)
        o2, S2 = fwd(q[t:], k[t:], v[t:], la[t:], b[t:], w[t:], S1)
        close(np.concatenate([o1, o2]), o, 1e-12, 'split output')
        close(S2, ST, 1e-12, 'split state')


def pin_varlen_independence(fwd):
    """Packed sequences (cu_seqlens) equal separate runs, including an empty one."""
    rng = np.random.default_rng(24)
    lens = [17, 0, 64, 1, 45]
    H, dk, dv = 2, 6, 5
    T = sum(lens)
    q, k, v, la, b, w, _ = rand_inputs(rng, T, H, dk, dv)
    S0 = 0.3 * rng.standard_normal((len(lens), H, dk, dv))
    cu = np.r_[0, np.cumsum(lens)]
    o, ST = fwd(q, k, v, la, b, w, S0, cu_seqlens=cu)
    for i, L in enumerate(lens):
        s = slice(cu[i], cu[i + 1])
        oi, Si = fwd(q[s], k[s], v[s], la[s], b[s], w[s], S0[i:i + 1])
        close(o[s], oi, 0.0, f'sequence {i} output')
        close(ST[i], Si[0], 0.0, f'sequence {i} state')
    close(ST[1], S0[1], 0.0, 'empty sequence keeps S0')


ALL = [pin_dense_product, pin_hand_worked, pin_alpha_free_transposed, pin_kda_collapse,
       pin_gdn_collapse, pin_textbook_delta_rule, pin_linear_attention, pin_decay_closed_form,
       pin_exact_retrieval, pin_pure_erase, pin_preservation, pin_full_forget,
       pin_erase_spectrum, pin_state_passing, pin_varlen_independence]
