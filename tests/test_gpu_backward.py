"""GPU parity for the chunkwise backward (gdn2_chunk_bwd): every gradient
against the token-level gradient oracle (oracle/gdn2_oracle_bwd.c), on
seeded inputs, with the forward tolerance bar applied to each gradient:
fp32 inputs max-abs <= 1e-4, bf16 inputs max-abs <= 2e-2 x RMS(reference)."""
import numpy as np
import pytest

import gdn2_inputs as gi

pytestmark = pytest.mark.gpu

torch = pytest.importorskip('torch')
if not torch.cuda.is_available():
    pytest.skip('no GPU', allow_module_level=True)

import gated_delta_rule_wy_amd as gdn2  # noqa: E402
import oracle  # noqa: E402
from gpu_util import assert_close, dev, tdtype, threads  # noqa: E402

NAMES = ('q', 'k', 'v', 'log_alpha', 'b', 'w', 'S0')


def grads_gpu(p, dO, dST, S0=True):
    td = tdtype(p.dtype)
    lead = (p.B, -1, p.H)
    t = lambda x, d: dev(x, d).reshape(*lead, x.shape[-1])
    g = gdn2.chunk_bwd(t(p.q, td), t(p.k, td), t(p.v, td), t(p.log_alpha, torch.float32), t(p.b, td), t(p.w, td),
                       dev(p.S0, torch.float32) if (S0 and p.S0 is not None) else None, t(dO, torch.float32),
                       None if dST is None else dev(dST, torch.float32),
                       dev(p.cu_seqlens, torch.int32) if p.varlen else None)
    torch.cuda.synchronize()
    return {n: g[n].cpu().numpy() for n in NAMES}


def check(p, label, S0=True, with_dST=True, seed=7, la_scale=None, f32_rel=False):
    """Every gradient at the forward's bar. `la_scale`: for bf16 inputs at
    uniform extreme decay, d log_alpha and dS0 are instead held to 2e-2 x the
    RMS of q * dq, the scale of the gradients they are damped from (see
    test_very_strong_decay)."""
    rng = np.random.default_rng(seed)
    dO = rng.standard_normal((p.tokens, p.H, p.dv)).astype(np.float32)
    dST = rng.standard_normal((p.N, p.H, p.dk, p.dv)).astype(np.float32) if with_dST else None
    print(f'[{label}] N={p.N} tokens={p.tokens} H={p.H} dk={p.dk} dv={p.dv} {p.dtype}', flush=True)
    g = grads_gpu(p, dO, dST, S0)
    ref = oracle.backward(p.q, p.k, p.v, p.log_alpha, p.b, p.w, p.S0 if S0 else None, dO, dST,
                          cu_seqlens=p.cu_seqlens, nthreads=threads())
    for n in NAMES:
        x = g[n].reshape(ref[n].shape)
        if n in ('log_alpha', 'S0') and la_scale and p.dtype == 'bf16':
            scale = float(np.sqrt(np.mean(np.square(p.q * ref['q']))))
            err = float(np.max(np.abs(x - ref[n])))
            rms = float(np.sqrt(np.mean(np.square(ref[n]))))
            print(f'{label} d{n}: max abs err {err:.3e}; RMS(ref) {rms:.3e}, RMS(q dq) {scale:.3e}', flush=True)
            assert np.all(np.isfinite(x)) and err <= 2e-2 * scale, f'{label} d{n}: {err:.3e} > 2e-2 x {scale:.3e}'
        elif f32_rel and p.dtype == 'f32':
            # 1e-4 of the gradient's largest magnitude (at least 1e-4)
            err = float(np.max(np.abs(x - ref[n])))
            bar = 1e-4 * max(1.0, float(np.max(np.abs(ref[n]))))
            print(f'{label} d{n}: max abs err {err:.3e} (bar {bar:.3e})', flush=True)
            assert np.all(np.isfinite(x)) and err <= bar, f'{label} d{n}: {err:.3e} > {bar:.3e}'
        else:
            assert_close(x, ref[n], p.dtype, f'{label} d{n}')


@pytest.mark.parametrize('dt,dk,dv', [('bf16', 128, 128), ('bf16', 64, 32), ('bf16', 32, 16), ('bf16', 128, 64),
                                      ('f32', 16, 16), ('f32', 64, 64), ('f32', 128, 32), ('f32', 32, 128)])
def test_uniform_ragged_tail(dt, dk, dv):
    p = gi.prefill(90 + dk + dv, [200] * 2, H=2, dk=dk, dv=dv, dtype=dt, s0_std=0.05)
    check(p, f'uniform {dt} dk={dk} dv={dv}')


@pytest.mark.parametrize('dt', ['bf16', 'f32'])
def test_varlen_with_empty_and_short(dt):
    lens = [130, 1, 0, 77, 64, 2]
    p = gi.prefill(91, lens, H=4, dk=128 if dt == 'bf16' else 64, dv=64, dtype=dt, s0_std=0.05, uniform=False)
    check(p, f'varlen {dt}')


def test_no_initial_state_no_final_gradient():
    p = gi.prefill(92, [333] * 2, H=2, dk=128, dv=128, dtype='bf16')
    check(p, 'no S0, no dS_T', S0=False, with_dST=False)


@pytest.mark.parametrize('dt', ['bf16', 'f32'])
def test_strong_decay(dt):
    """log alpha = -5 per token: chunk-cumulative decay down to -320, handled
    by the 16-row block references (diagonal blocks around their middle)."""
    p = gi.prefill(93, [300], H=2, dk=64, dv=64, dtype=dt, s0_std=0.05)
    p.log_alpha = np.full_like(p.log_alpha, -5.0)
    check(p, f'strong decay {dt}')


@pytest.mark.parametrize('la', [-10.0, -20.0, 'mixed'])
@pytest.mark.parametrize('dt', ['bf16', 'f32'])
def test_very_strong_decay(dt, la):
    """log alpha of -10 and -20 per token, and a mix of -20 and mild decay
    per token and channel: diagonal blocks whose decay is too wide for the
    middle-row factors take the exact pairwise exponents.

    At uniform -10 (-20) per token two gradients are damped far below the
    others: the decay gradient, 2e4 (4.5e8) times smaller in RMS than the
    terms q dq and k dk whose difference it is (it gathers only the
    interactions across each token, each damped by that token's alpha), and
    dS0, which reaches the state only through the first tokens' factors
    e^{g_r} <= e^{-10}, values that f16 operands hold as subnormals. With bf16
    inputs these two are held to 2e-2 x RMS(q dq): finite and at their scale,
    not to a relative bar. The mixed case and -5 per token hold every
    gradient to the usual bar, and fp32 inputs do at uniform decay. In the
    mixed case with fp32 inputs the cumulative log decay of a chunk reaches
    about -600 while single steps are mild; fp32 cumulative sums there carry
    absolute rounding near 1e-4, so its gradients (up to 15 in magnitude) are
    held to 1e-4 of their largest magnitude."""
    p = gi.prefill(96, [300, 77], H=2, dk=64, dv=64, dtype=dt, s0_std=0.05, uniform=False)
    if la == 'mixed':
        rng = np.random.default_rng(961)
        strong = rng.random(p.log_alpha.shape) < 0.5
        p.log_alpha = np.where(strong, -20.0, -rng.random(p.log_alpha.shape)).astype(np.float32)
    else:
        p.log_alpha = np.full_like(p.log_alpha, la)
    check(p, f'decay {la} {dt}', la_scale=la != 'mixed', f32_rel=la == 'mixed')


def test_many_chains_two_tile_slices():
    """Enough chains that the passes take two 16-column tiles per workgroup."""
    p = gi.prefill(94, [130, 64, 1, 200, 77] * 8, H=8, dk=128, dv=128, dtype='bf16', s0_std=0.05, uniform=False)
    check(p, 'two tiles')


def test_long_sequence():
    p = gi.prefill(95, [8401], H=2, dk=128, dv=128, dtype='bf16', s0_std=0.02)
    check(p, 'long T=8401')


def test_full_size_t65536():
    """The T = 65536, H = 16, d = 128 prefill workload's backward."""
    c = gi.WORKLOADS['prefill_t65536']
    p = gi.prefill(c['seed'], [c['T']], H=c['H'], dk=c['dk'], dv=c['dv'], dtype=c['dtype'], s0_std=c['s0_std'],
                   threads=threads())
    check(p, 'T=65536 H=16')


def test_deterministic():
    """Two runs on the same inputs give the same gradients bit for bit (the
    per-channel sums over a chunk's rows are taken in a fixed order)."""
    p = gi.prefill(97, [300, 77, 200], H=4, dk=128, dv=128, dtype='bf16', s0_std=0.05, uniform=False)
    rng = np.random.default_rng(5)
    dO = rng.standard_normal((p.tokens, p.H, p.dv)).astype(np.float32)
    dST = rng.standard_normal((p.N, p.H, p.dk, p.dv)).astype(np.float32)
    a = grads_gpu(p, dO, dST)
    b = grads_gpu(p, dO, dST)
    for n in NAMES:
        assert np.array_equal(a[n], b[n]), f'd{n} differs between two runs'
