"""GPU parity for the fused prologue (gdn2_chunk_fwd_prologue,
gdn2_decode_step_prologue): the mixer fed with raw q, k, v, which pass
through the short convolution (and unit norm for q and k) inside the
kernels, and with gate logits, which pass through the sigmoid there. The
oracle runs the same prologue in fp64 (oracle/prologue.py), then the
recurrence. The convolution history that comes back is a copy of raw inputs,
so it must match bit for bit."""
import numpy as np
import pytest

import gdn2_inputs as gi

pytestmark = pytest.mark.gpu

torch = pytest.importorskip('torch')
if not torch.cuda.is_available():
    pytest.skip('no GPU', allow_module_level=True)

import gated_delta_rule_wy_amd as gdn2  # noqa: E402
import oracle.prologue as opro  # noqa: E402
from gpu_util import assert_close, dev, tdtype, threads  # noqa: E402

QKV = ('q', 'k', 'v')


def _dev_triple(d, dtype):
    return None if d is None else tuple(dev(d[n], dtype) for n in QKV)


def run_prologue(p: gi.PrologueBatch, history=True, inplace=False, S0=True):
    dt = tdtype(p.dtype)
    lead = (p.B, -1, p.H)
    t = lambda x, d: dev(x, d).reshape(*lead, x.shape[-1])
    qr, kr, vr, xb, xw = (t(x, dt) for x in (p.q_raw, p.k_raw, p.v_raw, p.b_logit, p.w_logit))
    la = t(p.log_alpha, torch.float32)
    cw = _dev_triple(p.conv_w, torch.float32)
    cb = _dev_triple(p.conv_b, torch.float32)
    hin = _dev_triple(p.conv_in, dt) if history else None
    s0 = dev(p.S0, torch.float32) if (S0 and p.S0 is not None) else None
    cu = dev(p.cu_seqlens, torch.int32) if p.varlen else None
    o, ST, hout = gdn2.chunk_fwd_prologue(qr, kr, vr, la, xb, xw, cw, cb, s0, cu, conv_state=hin,
                                          conv_state_out=hin if inplace else None)
    torch.cuda.synchronize()
    hist = {n: h.float().cpu().numpy() for n, h in zip(QKV, hout)}
    return o.reshape(-1, p.H, p.dv).cpu().numpy(), ST.cpu().numpy(), hist


def oracle_run(p: gi.PrologueBatch, history=True, S0=True):
    return opro.forward_prologue(p.q_raw, p.k_raw, p.v_raw, p.conv_w, p.conv_b, p.log_alpha, p.b_logit,
                                 p.w_logit, S0=p.S0 if S0 else None, cu_seqlens=p.cu_seqlens,
                                 conv_in=p.conv_in if history else None, nthreads=threads())


def check(p, label, history=True, inplace=False, S0=True):
    print(f'[{label}] N={p.N} tokens={p.tokens} H={p.H} dk={p.dk} dv={p.dv} {p.dtype} '
          f'history={history and p.conv_in is not None} inplace={inplace}', flush=True)
    o, ST, hist = run_prologue(p, history, inplace, S0)
    o_ref, ST_ref, hist_ref = oracle_run(p, history, S0)
    assert_close(o, o_ref, p.dtype, f'{label} o')
    assert_close(ST, ST_ref, p.dtype, f'{label} S_T')
    for n in QKV:
        assert np.array_equal(hist[n], hist_ref[n].astype(np.float32)), f'{label}: history of {n} differs'


@pytest.mark.parametrize('dt,dk,dv', [('bf16', 128, 128), ('bf16', 64, 32), ('bf16', 32, 128),
                                      ('f32', 16, 16), ('f32', 64, 64), ('f32', 128, 16)])
def test_uniform_ragged_tail(dt, dk, dv):
    p = gi.prologue_prefill(60 + dk + dv, [200] * 2, H=2, dk=dk, dv=dv, dtype=dt, s0_std=0.05)
    check(p, f'uniform {dt} dk={dk} dv={dv}')


@pytest.mark.parametrize('dt', ['bf16', 'f32'])
def test_varlen_with_history(dt):
    """Packed sequences (some shorter than the history, one empty) continuing
    from a convolution history and S0."""
    lens = [130, 1, 0, 2, 77, 64, 200, 3]
    p = gi.prologue_prefill(71, lens, H=4, dk=128 if dt == 'bf16' else 64, dv=64, dtype=dt, s0_std=0.05,
                            uniform=False, conv_history=True)
    check(p, f'varlen history {dt}')


def test_history_updated_in_place():
    p = gi.prologue_prefill(72, [1, 5, 66, 2, 130], H=3, dk=128, dv=128, dtype='bf16', s0_std=0.05,
                            uniform=False, conv_history=True)
    check(p, 'in place', inplace=True)


def test_no_bias_no_history_no_s0():
    p = gi.prologue_prefill(73, [333] * 3, H=2, dk=64, dv=128, dtype='bf16', conv_bias=False)
    check(p, 'no bias', history=False, S0=False)


def test_two_tile_slices():
    """Enough chains that the pass takes two 16-column tiles per workgroup."""
    p = gi.prologue_prefill(74, [130, 64, 1, 200, 77] * 8, H=8, dk=128, dv=128, dtype='bf16', s0_std=0.05,
                            uniform=False, conv_history=True)
    check(p, 'two tiles')


@pytest.mark.parametrize('dt,dk,T', [('bf16', 128, 8401), ('f32', 64, 4159)])
def test_long_few_chains(dt, dk, T):
    """Long sequences over few chains (the prefetch workgroups are active)."""
    p = gi.prologue_prefill(75, [T], H=2, dk=dk, dv=dk, dtype=dt, s0_std=0.02, conv_history=True)
    check(p, f'long {dt} T={T}')


def test_full_size_t65536():
    """The T = 65536, H = 16, d = 128 workload in its raw (pre-prologue) form."""
    p = gi.prologue_prefill(76, [65536], H=16, dk=128, dv=128, dtype='bf16', s0_std=0.02, threads=threads())
    check(p, 'T=65536 H=16')


@pytest.mark.parametrize('dt,dk,dv,history', [('bf16', 128, 128, True), ('bf16', 64, 32, False),
                                              ('f32', 16, 64, True), ('f32', 128, 128, True)])
def test_decode_steps(dt, dk, dv, history):
    """Several decode steps with the history carried in place, against the
    oracle's step-by-step prologue and recurrence."""
    N, H = 8, 4
    S_np, h_np = gi.prologue_decode_state(80, N, H, dk, dv, dt)
    cw_np, cb_np = gi.conv_params(80, H, dk, dv)
    tdt = tdtype(dt)
    S = dev(S_np, torch.float32)
    hist = tuple(dev(h_np[n], tdt) for n in QKV) if history else None
    cw, cb = _dev_triple(cw_np, torch.float32), _dev_triple(cb_np, torch.float32)
    S_ref = S_np.astype(np.float64)
    h_ref = {n: h_np[n].astype(np.float64) for n in QKV} if history else None
    for s in range(1, 6):
        x = gi.prologue_decode_step(80, s, N, H, dk, dv, dt)
        qr, kr, vr, xb, xw = (dev(a, tdt) for a in (x[0], x[1], x[2], x[4], x[5]))
        la = dev(x[3], torch.float32)
        o = gdn2.decode_step_prologue(qr, kr, vr, la, xb, xw, S, cw, cb, hist)
        torch.cuda.synchronize()
        o_ref, S_ref, h_new = opro.decode_step_prologue(x[0], x[1], x[2], cw_np, cb_np, x[3], x[4], x[5], S_ref,
                                                        h_ref, nthreads=threads())
        print(f'[decode {dt} dk={dk} dv={dv}] step {s}', flush=True)
        assert_close(o.cpu().numpy(), o_ref, dt, f'decode step {s} o')
        assert_close(S.cpu().numpy(), S_ref, dt, f'decode step {s} S')
        if history:
            h_ref = h_new
            for n, h in zip(QKV, hist):
                assert np.array_equal(h.float().cpu().numpy(), h_ref[n].astype(np.float32)), f'history {n}'


def test_prefill_then_decode_continues():
    """A prefill's final state and history feed decode steps that continue the
    same sequences: equal to the oracle over the whole token range."""
    N, H, dk, dv, T, steps = 3, 2, 128, 64, 150, 4
    p = gi.prologue_prefill(81, [T + steps] * N, H=H, dk=dk, dv=dv, dtype='bf16', s0_std=0.02)
    o_ref, ST_ref, _ = oracle_run(p)
    o_ref = o_ref.reshape(N, T + steps, H, dv)
    head = gi.PrologueBatch(**{**p.__dict__})
    cut = lambda a: np.ascontiguousarray(a.reshape(N, T + steps, H, -1)[:, :T].reshape(N * T, H, -1))
    for name in ('q_raw', 'k_raw', 'v_raw', 'log_alpha', 'b_logit', 'w_logit'):
        setattr(head, name, cut(getattr(p, name)))
    head.T = T
    head.cu_seqlens = (np.arange(N + 1) * T).astype(np.int32)
    o, ST, hist = run_prologue(head)
    tdt = torch.bfloat16
    S = dev(ST, torch.float32)
    hcur = tuple(dev(hist[n], tdt) for n in QKV)
    cw, cb = _dev_triple(p.conv_w, torch.float32), _dev_triple(p.conv_b, torch.float32)
    tok = lambda a, s: np.ascontiguousarray(a.reshape(N, T + steps, H, -1)[:, T + s])
    for s in range(steps):
        args = [dev(tok(getattr(p, n), s), tdt) for n in ('q_raw', 'k_raw', 'v_raw')]
        la = dev(tok(p.log_alpha, s), torch.float32)
        xb, xw = dev(tok(p.b_logit, s), tdt), dev(tok(p.w_logit, s), tdt)
        od = gdn2.decode_step_prologue(*args, la, xb, xw, S, cw, cb, hcur)
        torch.cuda.synchronize()
        assert_close(od.cpu().numpy(), o_ref[:, T + s], 'bf16', f'continued decode step {s}')
    assert_close(S.cpu().numpy(), ST_ref, 'bf16', 'final state after prefill + decode')
