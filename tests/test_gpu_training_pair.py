"""GPU tests of the training pair (gdn2_chunk_fwd_keep, gdn2_chunk_bwd_kept):
the forward that keeps what the backward needs returns o and S_T equal bit
for bit to gdn2_chunk_fwd, and the backward from what it kept returns
gradients equal bit for bit to gdn2_chunk_bwd (which runs the forward again
itself); one case is also held against the gradient oracle at the forward's
bar (bf16 inputs: max-abs <= 2e-2 x RMS(reference); fp32: <= 1e-4)."""
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


def tensors(p, seed=7, S0=True):
    td = tdtype(p.dtype)
    lead = (p.B, -1, p.H)
    t = lambda x, d: dev(x, d).reshape(*lead, x.shape[-1])
    rng = np.random.default_rng(seed)
    dO = rng.standard_normal((p.tokens, p.H, p.dv)).astype(np.float32)
    dST = rng.standard_normal((p.N, p.H, p.dk, p.dv)).astype(np.float32)
    return dict(q=t(p.q, td), k=t(p.k, td), v=t(p.v, td), log_alpha=t(p.log_alpha, torch.float32),
                b=t(p.b, td), w=t(p.w, td),
                S0=dev(p.S0, torch.float32) if (S0 and p.S0 is not None) else None,
                cu=dev(p.cu_seqlens, torch.int32) if p.varlen else None,
                dO=t(dO, torch.float32), dST=dev(dST, torch.float32)), dO, dST


def run_pair(p, label, S0=True):
    """chunk_fwd_keep + chunk_bwd_kept against chunk_fwd and chunk_bwd."""
    x, dO, dST = tensors(p, S0=S0)
    print(f'[{label}] N={p.N} tokens={p.tokens} H={p.H} dk={p.dk} dv={p.dv} {p.dtype}', flush=True)
    args = (x['q'], x['k'], x['v'], x['log_alpha'], x['b'], x['w'], x['S0'])
    o_ref, ST_ref = gdn2.chunk_fwd(*args, x['cu'])
    g_ref = gdn2.chunk_bwd(*args, x['dO'], x['dST'], x['cu'])
    o, ST, ws = gdn2.chunk_fwd_keep(*args, x['cu'])
    g = gdn2.chunk_bwd_kept(*args, x['dO'], x['dST'], x['cu'], workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref), f'{label}: o differs from chunk_fwd'
    assert torch.equal(ST, ST_ref), f'{label}: S_T differs from chunk_fwd'
    for n in NAMES:
        assert torch.equal(g[n], g_ref[n]), f'{label}: d{n} differs from chunk_bwd'
    return g, dO, dST


@pytest.mark.parametrize('dt,dk,dv', [('bf16', 128, 128), ('bf16', 64, 32), ('f32', 64, 64), ('f32', 16, 16)])
def test_pair_equals_separate_calls(dt, dk, dv):
    p = gi.prefill(700 + dk + dv, [200] * 2, H=2, dk=dk, dv=dv, dtype=dt, s0_std=0.05)
    run_pair(p, f'uniform {dt} dk={dk} dv={dv}')


def test_pair_varlen_with_empty_and_short():
    p = gi.prefill(711, [130, 1, 0, 77, 64, 2], H=4, dk=128, dv=64, dtype='bf16', s0_std=0.05, uniform=False)
    run_pair(p, 'varlen')


def test_pair_two_tile_slices():
    """Enough chains that the passes take two 16-column tiles per workgroup."""
    p = gi.prefill(712, [130, 64, 1, 200, 77] * 8, H=8, dk=128, dv=128, dtype='bf16', s0_std=0.05, uniform=False)
    run_pair(p, 'two tiles')


def test_pair_no_initial_state():
    p = gi.prefill(713, [333] * 2, H=2, dk=128, dv=128, dtype='bf16')
    run_pair(p, 'no S0', S0=False)


def test_pair_against_oracle():
    p = gi.prefill(714, [300, 77], H=2, dk=128, dv=128, dtype='bf16', s0_std=0.05, uniform=False)
    g, dO, dST = run_pair(p, 'oracle')
    ref = oracle.backward(p.q, p.k, p.v, p.log_alpha, p.b, p.w, p.S0, dO, dST, cu_seqlens=p.cu_seqlens,
                          nthreads=threads())
    for n in NAMES:
        assert_close(g[n].cpu().numpy().reshape(ref[n].shape), ref[n], p.dtype, f'kept backward d{n}')


def test_pair_reused_workspace():
    """Two training steps on one workspace, the second with other inputs:
    the backward follows the latest forward."""
    p1 = gi.prefill(715, [256], H=2, dk=128, dv=128, dtype='bf16', s0_std=0.05)
    p2 = gi.prefill(716, [256], H=2, dk=128, dv=128, dtype='bf16', s0_std=0.05)
    x1, _, _ = tensors(p1)
    x2, _, _ = tensors(p2, seed=8)
    a1 = (x1['q'], x1['k'], x1['v'], x1['log_alpha'], x1['b'], x1['w'], x1['S0'])
    a2 = (x2['q'], x2['k'], x2['v'], x2['log_alpha'], x2['b'], x2['w'], x2['S0'])
    _, _, ws = gdn2.chunk_fwd_keep(*a1)
    gdn2.chunk_bwd_kept(*a1, x1['dO'], x1['dST'], workspace=ws)
    gdn2.chunk_fwd_keep(*a2, workspace=ws)
    g = gdn2.chunk_bwd_kept(*a2, x2['dO'], x2['dST'], workspace=ws)
    g_ref = gdn2.chunk_bwd(*a2, x2['dO'], x2['dST'])
    torch.cuda.synchronize()
    for n in NAMES:
        assert torch.equal(g[n], g_ref[n]), f'second step: d{n} differs from chunk_bwd'


def test_pair_full_size_t65536():
    """The T = 65536, H = 16, d = 128 prefill workload, in the launch
    configuration the training step is timed in."""
    c = gi.WORKLOADS['prefill_t65536']
    p = gi.prefill(c['seed'], [c['T']], H=c['H'], dk=c['dk'], dv=c['dv'], dtype=c['dtype'], s0_std=c['s0_std'],
                   threads=threads())
    run_pair(p, 'T=65536 H=16')
