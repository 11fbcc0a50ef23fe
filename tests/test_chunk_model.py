"""The chunkwise WY algebra (fp64 model) reproduces the oracle exactly (CPU)."""
import numpy as np
import pytest

import chunk_model
import oracle
import pins


@pytest.mark.parametrize('C', [1, 16, 64])
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
    o, ST = chunk_model.chunk_forward(q, k, v, la, b, w, S0)
    pins.close(o, o_ref, 1e-12, 'strong decay o')
    pins.close(ST, ST_ref, 1e-12, 'strong decay S_T')
