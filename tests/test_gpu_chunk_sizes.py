"""GPU parity for the chunk-size variants (gdn2_chunk_fwd_sized, chunks of 32
and 128 tokens) against the fp64 oracle, with the bars of the 64-token path:
fp32 inputs max-abs <= 1e-4; bf16 inputs max-abs <= 2e-2 x RMS(reference).
The oracle is the token recurrence, so it does not depend on the chunk size."""
import numpy as np
import pytest

import gdn2_inputs as gi

pytestmark = pytest.mark.gpu

torch = pytest.importorskip('torch')
if not torch.cuda.is_available():
    pytest.skip('no GPU', allow_module_level=True)

import gated_delta_rule_wy_amd as gdn2  # noqa: E402
from gpu_util import assert_close, oracle_prefill, run_prefill  # noqa: E402

CHUNKS = [32, 128]


def check(p, C, label, **kw):
    print(f'[C={C} {label}] N={p.N} tokens={p.tokens} H={p.H} dk={p.dk} dv={p.dv} {p.dtype}', flush=True)
    o, ST = run_prefill(p, chunk=C, **kw)
    o_ref, ST_ref = oracle_prefill(p)
    assert_close(o, o_ref, p.dtype, f'C={C} {label} o')
    if ST is not None:
        assert_close(ST, ST_ref, p.dtype, f'C={C} {label} S_T')
    return o, ST


@pytest.mark.parametrize('C', CHUNKS)
@pytest.mark.parametrize('dt,dk,dv', [('bf16', 128, 128), ('bf16', 64, 32), ('bf16', 32, 16), ('bf16', 128, 64),
                                      ('f32', 16, 16), ('f32', 64, 64), ('f32', 32, 128)])
@pytest.mark.parametrize('T', [1, 31, 33, 128, 129, 300])
def test_shapes_ragged(C, dt, dk, dv, T):
    """Lengths around both chunk sizes, packed with a second, shorter sequence."""
    p = gi.prefill(1100 + T + dk + dv, [T, max(1, T // 3)], H=2, dk=dk, dv=dv, dtype=dt, s0_std=0.05,
                   uniform=False)
    check(p, C, f'{dt} dk={dk} dv={dv} T={T}')


def test_f32_dk128_chunk32():
    p = gi.prefill(1150, [200, 77], H=2, dk=128, dv=32, dtype='f32', s0_std=0.05, uniform=False)
    check(p, 32, 'f32 dk=128 dv=32')


def test_f32_dk128_chunk128_unsupported():
    """The 128-token prep's tiles do not fit one compute unit's LDS for fp32
    inputs at dk = 128: the call is refused before any launch."""
    p = gi.prefill(1151, [100], H=1, dk=128, dv=32, dtype='f32', s0_std=0.05, uniform=False)
    with pytest.raises(gdn2.Gdn2Error) as e:
        run_prefill(p, chunk=128)
    assert e.value.status == gdn2.GDN2_ERR_UNSUPPORTED


@pytest.mark.parametrize('C', CHUNKS)
@pytest.mark.parametrize('dt', ['bf16', 'f32'])
def test_varlen_edges(C, dt):
    """Empty sequences keep S0; lengths at and around both chunk sizes."""
    lens = [0, 1, 32, 0, 33, 128, 127, 129, 3, 0, 64]
    p = gi.prefill(1200, lens, H=2, dk=128 if dt == 'bf16' else 32, dv=64, dtype=dt, s0_std=0.05, uniform=False)
    o, ST = check(p, C, f'varlen edges {dt}')
    for i, L in enumerate(lens):
        if L == 0:
            assert np.array_equal(ST[i], p.S0[i]), 'empty sequence must return S0 unchanged'


@pytest.mark.parametrize('C', CHUNKS)
@pytest.mark.parametrize('dt', ['bf16', 'f32'])
def test_strong_decay(C, dt):
    """log alpha = -5 per token: every diagonal block takes the exact
    (pairwise-exponent) path and the off-diagonal blocks the row-block references."""
    p = gi.prefill(1300, [300, 128, 37], H=2, dk=128 if dt == 'bf16' else 64, dv=64, dtype=dt, s0_std=0.02,
                   uniform=False)
    p.log_alpha[:] = -5.0
    check(p, C, f'strong decay {dt}')


@pytest.mark.parametrize('C', CHUNKS)
def test_mixed_decay_rates(C):
    """Strong decay in a few channels and tokens (mixes the fast and slow chunk paths)."""
    p = gi.prefill(1301, [400], H=2, dk=128, dv=128, dtype='bf16', s0_std=0.02, uniform=False)
    rng = np.random.default_rng(1)
    p.log_alpha[rng.random(p.log_alpha.shape) < 0.05] = -8.0
    check(p, C, 'mixed decay')


@pytest.mark.parametrize('C', CHUNKS)
@pytest.mark.parametrize('dt,dk,dv', [('bf16', 128, 128), ('f32', 64, 32)])
def test_many_chains_two_tile_slices(C, dt, dk, dv):
    """Enough chains that the pass takes two 16-column tiles per workgroup."""
    lens = [130, 64, 1, 200, 77] * 8
    p = gi.prefill(1400 + C, lens, H=8, dk=dk, dv=dv, dtype=dt, s0_std=0.05, uniform=False)
    check(p, C, f'two-tile {dt}')


@pytest.mark.parametrize('C', CHUNKS)
@pytest.mark.parametrize('dt,d,T', [('bf16', 128, 8401), ('f32', 64, 4159)])
def test_long_few_chains(C, dt, d, T):
    """Long sequences over few chains: the pass runs with its L2 prefetch workgroups."""
    p = gi.prefill(1500 + T, [T], H=2, dk=d, dv=d, dtype=dt, s0_std=0.05, uniform=True)
    check(p, C, f'long {dt} T={T}')


@pytest.mark.parametrize('C', CHUNKS)
def test_no_s0_no_final_state(C):
    p = gi.prefill(1600, [1000], H=2, dk=128, dv=128, dtype='bf16', s0_std=0.0, uniform=True)
    check(p, C, 'no S0, no S_T', output_final_state=False)


@pytest.mark.parametrize('C', CHUNKS)
def test_deterministic_and_same_recurrence(C):
    """Run to run bitwise identical; and within the bar of the 64-token path."""
    p = gi.prefill(1700, [333, 100], H=4, dk=128, dv=128, dtype='bf16', s0_std=0.02, uniform=False)
    o1, s1 = run_prefill(p, chunk=C)
    o2, s2 = run_prefill(p, chunk=C)
    assert np.array_equal(o1, o2) and np.array_equal(s1, s2), 'run-to-run results differ'
    o64, s64 = run_prefill(p)
    assert_close(o1, o64, 'bf16', f'C={C} vs C=64 o')
    assert_close(s1, s64, 'bf16', f'C={C} vs C=64 S_T')


@pytest.mark.parametrize('C', CHUNKS)
def test_full_size_t65536(C):
    """The T = 65536, H = 16, d = 128 prefill workload at this chunk size."""
    c = gi.WORKLOADS['prefill_t65536']
    from gpu_util import threads
    p = gi.prefill(c['seed'], [c['T']], H=c['H'], dk=c['dk'], dv=c['dv'], dtype=c['dtype'], s0_std=c['s0_std'],
                   threads=threads())
    check(p, C, 'T=65536 H=16')


@pytest.mark.parametrize('C', [32, 64, 128])
@pytest.mark.parametrize('dk,dv', [(64, 32), (128, 128), (32, 16)])
def test_repeat_is_bitwise_identical(C, dk, dv):
    """The pass has no data race: two calls on the same inputs give the same
    bits (a branch after a matrix instruction once gave states that varied
    from run to run at dk = 64)."""
    p = gi.prefill(1500 + C + dk, [300, 100], H=2, dk=dk, dv=dv, dtype='bf16', s0_std=0.05, uniform=False)
    o1, S1 = run_prefill(p, chunk=C)
    o2, S2 = run_prefill(p, chunk=C)
    assert np.array_equal(o1, o2) and np.array_equal(S1, S2)
    o_ref, S_ref = oracle_prefill(p)
    assert_close(o1, o_ref, p.dtype, f'C={C} dk={dk} dv={dv} o')
