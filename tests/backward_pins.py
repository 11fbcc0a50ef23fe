"""Pins for the gradient oracle (oracle/gdn2_oracle_bwd.c).

Each pin takes a backward callable with the signature of ``oracle.backward``
(so the same pins can run against copies with planted mistakes, see
test_oracle_mutants.py) and checks it against something other than itself:

* central finite differences of the pinned forward oracle (the loss is
  sum(dO * o) + sum(dS_T * S_T)), on every input element;
* closed forms for the linear-attention case (b = 0, alpha = 1), where the
  recurrence is a running sum and each gradient is a few matrix products;
* properties the gradients of the recurrence must have: o and S_T are affine
  in S0 (so dS0 does not depend on S0), a split sequence with the state and
  its gradient carried equals the whole, packed sequences are independent,
  and a full forget (alpha = 0) cuts the gradient to S0.

The forward recurrence is the Gated Delta Rule-2 (snilld.dk, "Hvad Gated
DeltaNet-2 ændrer", update equation) with readout after the update
(aifetchly-blog.pages.dev, "Gated DeltaNet-2 Guide", layer workflow step 4).
"""
from __future__ import annotations

import numpy as np

import oracle

NAMES = ('q', 'k', 'v', 'log_alpha', 'b', 'w')


def rand_problem(rng, lens, H, dk, dv, s0=0.4):
    n = int(sum(lens))
    x = dict(q=rng.standard_normal((n, H, dk)), k=rng.standard_normal((n, H, dk)) * 0.6,
             v=rng.standard_normal((n, H, dv)),
             log_alpha=-np.logaddexp(0, rng.standard_normal((n, H, dk)) - 1.0),
             b=1 / (1 + np.exp(-rng.standard_normal((n, H, dk)))),
             w=1 / (1 + np.exp(-rng.standard_normal((n, H, dv)))))
    N = len(lens)
    S0 = s0 * rng.standard_normal((N, H, dk, dv))
    dO = rng.standard_normal((n, H, dv))
    dST = rng.standard_normal((N, H, dk, dv))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    return x, S0, dO, dST, cu


def loss(x, S0, dO, dST, cu):
    o, ST = oracle.forward(x['q'], x['k'], x['v'], x['log_alpha'], x['b'], x['w'], S0, cu_seqlens=cu)
    return float(np.sum(o * dO) + np.sum(ST * dST))


def _close(a, b, tol, what):
    err = float(np.max(np.abs(np.asarray(a) - np.asarray(b)))) if np.size(a) else 0.0
    assert err <= tol, f'{what}: max abs diff {err:.3e} > {tol:.1e}'


def pin_finite_differences(bwd):
    """Every gradient against central differences of the forward oracle,
    over packed sequences (one empty, one longer than the 64-token
    checkpoint interval)."""
    rng = np.random.default_rng(101)
    x, S0, dO, dST, cu = rand_problem(rng, [7, 0, 3, 70], H=2, dk=3, dv=2)
    g = bwd(x['q'], x['k'], x['v'], x['log_alpha'], x['b'], x['w'], S0, dO, dST, cu_seqlens=cu)
    h = 1e-6
    for name in NAMES + ('S0',):
        base = S0 if name == 'S0' else x[name]
        num = np.zeros_like(base)
        for idx in np.ndindex(base.shape):
            vals = []
            for sgn in (1, -1):
                pert = base.copy()
                pert[idx] += sgn * h
                if name == 'S0':
                    vals.append(loss(x, pert, dO, dST, cu))
                else:
                    vals.append(loss({**x, name: pert}, S0, dO, dST, cu))
            num[idx] = (vals[0] - vals[1]) / (2 * h)
        _close(g[name], num, 2e-7 * max(1.0, float(np.max(np.abs(num)))), f'd{name}')


def pin_linear_attention(bwd):
    """b = 0, alpha = 1: S_t = S0 + sum_{s<=t} k_s u_s^T and o_t = S_t^T q_t,
    so with G_s = sum_{t>=s} q_t dO_t^T + dS_T (the gradient at S_s):
    dq_t = S_t dO_t, dk_s = G_s u_s, du_s = G_s^T k_s, dS0 = G_1,
    db_s = -k_s * (S_{s-1} du_s), dlog_alpha_s = rowsum(G_s * S_{s-1})."""
    rng = np.random.default_rng(102)
    T, H, dk, dv = 11, 2, 4, 3
    x, S0, dO, dST, _ = rand_problem(rng, [T], H, dk, dv)
    x['b'] = np.zeros_like(x['b'])
    x['log_alpha'] = np.zeros_like(x['log_alpha'])
    g = bwd(x['q'], x['k'], x['v'], x['log_alpha'], x['b'], x['w'], S0, dO, dST)
    for h in range(H):
        K, Q, dOh = x['k'][:, h], x['q'][:, h], dO[:, h]
        U = x['w'][:, h] * x['v'][:, h]
        S = S0[0, h][None] + np.cumsum(K[:, :, None] * U[:, None, :], axis=0)     # S_t, t = 0..T-1
        Sprev = np.concatenate([S0[0, h][None], S[:-1]])
        G = np.cumsum((Q[:, :, None] * dOh[:, None, :])[::-1], axis=0)[::-1] + dST[0, h][None]
        du = np.einsum('tcj,tc->tj', G, K)
        _close(g['q'][:, h], np.einsum('tcj,tj->tc', S, dOh), 1e-12, 'dq')
        _close(g['k'][:, h], np.einsum('tcj,tj->tc', G, U), 1e-12, 'dk')
        _close(g['v'][:, h], du * x['w'][:, h], 1e-12, 'dv')
        _close(g['w'][:, h], du * x['v'][:, h], 1e-12, 'dw')
        _close(g['S0'][0, h], G[0], 1e-12, 'dS0')
        _close(g['b'][:, h], -K * np.einsum('tcj,tj->tc', Sprev, du), 1e-12, 'db')
        _close(g['log_alpha'][:, h], np.sum(G * Sprev, axis=2), 1e-12, 'dlog_alpha')


def pin_affine_in_S0(bwd):
    """o and S_T are affine in S0: dS0 and every other gradient's dependence
    on S0 is linear, so dS0 is the same for any S0."""
    rng = np.random.default_rng(103)
    x, S0, dO, dST, cu = rand_problem(rng, [9, 4], H=2, dk=3, dv=3)
    g1 = bwd(x['q'], x['k'], x['v'], x['log_alpha'], x['b'], x['w'], S0, dO, dST, cu_seqlens=cu)
    g2 = bwd(x['q'], x['k'], x['v'], x['log_alpha'], x['b'], x['w'], 3.0 * S0 + 1.0, dO, dST, cu_seqlens=cu)
    _close(g1['S0'], g2['S0'], 1e-12, 'dS0 independent of S0')


def pin_state_passing(bwd):
    """A sequence split at t: the second half runs from the first half's
    final state; the first half receives the second half's dS0 as its dS_T.
    The gradients equal those of one call over the whole sequence."""
    rng = np.random.default_rng(104)
    x, S0, dO, dST, _ = rand_problem(rng, [90], H=2, dk=3, dv=2)
    g = bwd(x['q'], x['k'], x['v'], x['log_alpha'], x['b'], x['w'], S0, dO, dST)
    for t in (1, 40, 64, 89):
        a, z = slice(0, t), slice(t, 90)
        _, Smid = oracle.forward(*(x[n][a] for n in NAMES), S0, want_o=False)
        g2 = bwd(*(x[n][z] for n in NAMES), Smid, dO[z], dST)
        g1 = bwd(*(x[n][a] for n in NAMES), S0, dO[a], g2['S0'])
        for n in NAMES:
            _close(np.concatenate([g1[n], g2[n]]), g[n], 1e-10, f'split at {t}: d{n}')
        _close(g1['S0'], g['S0'], 1e-10, f'split at {t}: dS0')


def pin_varlen_independence(bwd):
    """Packed sequences give the gradients of separate calls."""
    rng = np.random.default_rng(105)
    lens = [5, 1, 0, 12]
    x, S0, dO, dST, cu = rand_problem(rng, lens, H=2, dk=2, dv=3)
    g = bwd(x['q'], x['k'], x['v'], x['log_alpha'], x['b'], x['w'], S0, dO, dST, cu_seqlens=cu)
    for i in range(len(lens)):
        s = slice(int(cu[i]), int(cu[i + 1]))
        gi = bwd(*(x[n][s] for n in NAMES), S0[i:i + 1], dO[s], dST[i:i + 1])
        for n in NAMES:
            _close(g[n][s], gi[n], 1e-13, f'sequence {i}: d{n}')
        _close(g['S0'][i], gi['S0'][0], 1e-13, f'sequence {i}: dS0')


def pin_full_forget(bwd):
    """alpha = 0 at the first token erases S0 from everything after it, so
    dS0 = 0 exactly; the other gradients stay finite."""
    rng = np.random.default_rng(106)
    x, S0, dO, dST, _ = rand_problem(rng, [6], H=1, dk=3, dv=2)
    x['log_alpha'][0] = -np.inf
    g = bwd(x['q'], x['k'], x['v'], x['log_alpha'], x['b'], x['w'], S0, dO, dST)
    assert np.all(g['S0'] == 0.0), 'dS0 must vanish after a full forget'
    for n in NAMES:
        if n != 'log_alpha':
            assert np.all(np.isfinite(g[n])), f'd{n} not finite'


ALL = [pin_finite_differences, pin_linear_attention, pin_affine_in_S0, pin_state_passing,
       pin_varlen_independence, pin_full_forget]
