"""The oracle against its pins (CPU only)."""
import numpy as np
import pytest

import oracle
import pins


def oracle_fwd(q, k, v, la, b, w, S0=None, cu_seqlens=None, B=None):
    return oracle.forward(q, k, v, la, b, w, S0, cu_seqlens=cu_seqlens, B=B)


@pytest.mark.parametrize('pin', pins.ALL, ids=[p.__name__ for p in pins.ALL])
def test_pin(pin):
    pin(oracle_fwd)


def test_decode_steps_equal_forward():
    """T single-token decode steps reproduce the forward over T tokens (state carried)."""
    rng = np.random.default_rng(30)
    N, H, dk, dv, T = 3, 2, 8, 6, 25
    q, k, v, la, b, w, _ = pins.rand_inputs(rng, N * T, H, dk, dv)
    S0 = 0.3 * rng.standard_normal((N, H, dk, dv))
    # tokens laid out sequence-major for the forward: [N, T, H, d]
    r = lambda x: x.reshape(N, T, H, -1)
    o_ref, ST_ref = oracle.forward(*(r(x) for x in (q, k, v, la, b, w)), S0)
    o_ref = o_ref.reshape(N, T, H, dv)
    S = S0.copy()
    for t in range(T):
        o, S = oracle.decode_step(*(r(x)[:, t] for x in (q, k, v, la, b, w)), S)
        pins.close(o, o_ref[:, t], 1e-12, f'decode step {t}')
    pins.close(S, ST_ref, 1e-12, 'decode final state')


def test_decode_step_dense():
    """One decode step against the printed dense update."""
    rng = np.random.default_rng(31)
    N, H, dk, dv = 4, 3, 7, 5
    q, k, v, la, b, w, _ = pins.rand_inputs(rng, N, H, dk, dv)
    S0 = 0.3 * rng.standard_normal((N, H, dk, dv))
    o, S1 = oracle.decode_step(q, k, v, la, b, w, S0)
    for n in range(N):
        for h in range(H):
            M = (np.eye(dk) - np.outer(k[n, h], b[n, h] * k[n, h])) @ np.diag(np.exp(la[n, h]))
            S_ref = M @ S0[n, h] + np.outer(k[n, h], w[n, h] * v[n, h])
            pins.close(S1[n, h], S_ref, 1e-12, 'decode state')
            pins.close(o[n, h], S_ref.T @ q[n, h], 1e-12, 'decode readout')


def test_threads_do_not_change_results():
    rng = np.random.default_rng(32)
    q, k, v, la, b, w, _ = pins.rand_inputs(rng, 4 * 40, 3, 8, 8)
    a = oracle.forward(q, k, v, la, b, w, B=4, nthreads=1)
    c = oracle.forward(q, k, v, la, b, w, B=4, nthreads=5)
    assert np.array_equal(a[0], c[0]) and np.array_equal(a[1], c[1])


import oracle.prologue as prologue_oracle
import prologue_pins


@pytest.mark.parametrize('pin', prologue_pins.ALL, ids=[p.__name__ for p in prologue_pins.ALL])
def test_prologue_pin(pin):
    pin(prologue_oracle)


import backward_pins


@pytest.mark.parametrize('pin', backward_pins.ALL, ids=[p.__name__ for p in backward_pins.ALL])
def test_backward_pin(pin):
    pin(oracle.backward)
