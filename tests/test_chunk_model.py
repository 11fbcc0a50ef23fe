"""The chunkwise WY algebra (fp64 model) reproduces the oracle exactly (CPU)."""
import numpy as np
import pytest

import chunk_model
import oracle
import pins


@pytest.mark.parametrize('C', [1, 16, 32, 64, 128])
def test_chunk_form_equals_oracle(C):
    rng = np.random.default_rng(40 + C)
    lens = [130, 64, 1, 0, 77]
    H, dk, dv = 2, 16, 12
    T = sum(lens)
    q, k, v, la, b, w, _ = pins.rand_inputs(rng, T, H, dk, dv)
    S0 = 0.3 * rng.standard_normal((len(lens), H, dk, dv))
    cu = np.r_[0, np.cumsum(lens)]
    o_ref, ST_ref = oracle.forward(q, k, v, la, b, w, S0, cu_seqlens=cu)
    o, ST = chunk_model.chunk_forward(q, k, v, la, b, w, S0, cu, C=C)
    pins.close(o, o_ref, 1e-12, 'chunk-form o')
    pins.close(ST, ST_ref, 1e-12, 'chunk-form S_T')


def test_chunk_form_strong_decay():
    """Per-token log alpha = -5 (chunk-cumulative decay down to -320): the
    pairwise exponents g_r - g_s <= 0 keep the chunk form exact."""
    rng = np.random.default_rng(50)
    T, H, dk, dv = 200, 1, 8, 8
    q, k, v, la, b, w, S0 = pins.rand_inputs(rng, T, H, dk, dv)
    la = np.full_like(la, -5.0)
    o_ref, ST_ref = oracle.forward(q, k, v, la, b, w, S0)
    for C in (32, 64, 128):
        o, ST = chunk_model.chunk_forward(q, k, v, la, b, w, S0, C=C)
        pins.close(o, o_ref, 1e-12, f'strong decay o, C={C}')
        pins.close(ST, ST_ref, 1e-12, f'strong decay S_T, C={C}')


@pytest.mark.parametrize('C', [1, 16, 64])
def test_chunk_backward_equals_oracle(C):
    """The chunk-form gradients (per chunk: dDelta, dX, dA, dP, then through
    the decay factors) equal the token-level gradient oracle."""
    rng = np.random.default_rng(60 + C)
    lens = [130, 64, 1, 0, 77]
    H, dk, dv = 2, 16, 12
    T = sum(lens)
    q, k, v, la, b, w, _ = pins.rand_inputs(rng, T, H, dk, dv)
    S0 = 0.3 * rng.standard_normal((len(lens), H, dk, dv))
    dO = rng.standard_normal((T, H, dv))
    dST = rng.standard_normal((len(lens), H, dk, dv))
    cu = np.r_[0, np.cumsum(lens)]
    ref = oracle.backward(q, k, v, la, b, w, S0, dO, dST, cu_seqlens=cu)
    got = chunk_model.chunk_backward(q, k, v, la, b, w, dO, S0, dST, cu, C=C)
    for n in ('q', 'k', 'v', 'log_alpha', 'b', 'w', 'S0'):
        pins.close(got[n], ref[n], 1e-10 * max(1.0, float(np.max(np.abs(ref[n])))), f'chunk-form d{n}')


def test_chunk_backward_strong_decay():
    rng = np.random.default_rng(70)
    T, H, dk, dv = 150, 1, 8, 8
    q, k, v, la, b, w, S0 = pins.rand_inputs(rng, T, H, dk, dv)
    la = np.full_like(la, -5.0)
    dO = rng.standard_normal((T, H, dv))
    dST = rng.standard_normal((1, H, dk, dv))
    ref = oracle.backward(q, k, v, la, b, w, S0, dO, dST)
    got = chunk_model.chunk_backward(q, k, v, la, b, w, dO, S0, dST)
    for n in ('q', 'k', 'v', 'log_alpha', 'b', 'w', 'S0'):
        pins.close(got[n], ref[n], 1e-10 * max(1.0, float(np.max(np.abs(ref[n])))), f'strong decay d{n}')
