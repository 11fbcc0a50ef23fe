"""GPU parity for the per-token-head gate layouts (gdn2_chunk_fwd_gates,
gdn2_decode_step_gates): Kimi Delta Attention (erase and write gates one
scalar beta per token-head) and Gated DeltaNet (also a scalar decay), the
special cases Gated DeltaNet-2 reduces to, plus each gate alone. The oracle
runs the same recurrence on the gates broadcast over their channels."""
import numpy as np
import pytest

import gdn2_inputs as gi

pytestmark = pytest.mark.gpu

torch = pytest.importorskip('torch')
if not torch.cuda.is_available():
    pytest.skip('no GPU', allow_module_level=True)

import gated_delta_rule_wy_amd as gdn2  # noqa: E402
import oracle  # noqa: E402
from gpu_util import DEV, assert_close, dev, oracle_prefill, tdtype, threads  # noqa: E402

KDA = gdn2.GDN2_GATE_B_PER_HEAD | gdn2.GDN2_GATE_W_PER_HEAD
GDN = KDA | gdn2.GDN2_GATE_ALPHA_PER_HEAD


def gated_batch(seed, lens, H, dk, dv, dt, gates, uniform, s0_std=0.05):
    """A batch whose per-head gates (where `gates` says so) are constant over
    channels: b = w = beta when both are per-head (KDA form)."""
    p = gi.prefill(seed, lens, H=H, dk=dk, dv=dv, dtype=dt, s0_std=s0_std, uniform=uniform)
    col = gi.prefill(seed, lens, H=H, dk=dk, dv=dv, dtype=dt, s0_std=s0_std, uniform=uniform, collapsed=H)
    beta = col.b[..., 0]
    if gates & gdn2.GDN2_GATE_B_PER_HEAD:
        p.b = np.ascontiguousarray(np.broadcast_to(beta[..., None], p.b.shape))
    if gates & gdn2.GDN2_GATE_W_PER_HEAD:
        p.w = np.ascontiguousarray(np.broadcast_to(beta[..., None], p.w.shape))
    if gates & gdn2.GDN2_GATE_ALPHA_PER_HEAD:
        p.log_alpha = np.ascontiguousarray(np.broadcast_to(col.log_alpha[..., :1], p.log_alpha.shape))
    return p


def run_gated(p, gates):
    dt = tdtype(p.dtype)
    lead = (p.B, -1, p.H)
    full = lambda x, d: dev(x, d).reshape(*lead, x.shape[-1])
    head = lambda x, d: dev(np.ascontiguousarray(x[..., 0]), d).reshape(*lead)
    q, k, v = (full(x, dt) for x in (p.q, p.k, p.v))
    b = head(p.b, dt) if gates & gdn2.GDN2_GATE_B_PER_HEAD else full(p.b, dt)
    w = head(p.w, dt) if gates & gdn2.GDN2_GATE_W_PER_HEAD else full(p.w, dt)
    la = head(p.log_alpha, torch.float32) if gates & gdn2.GDN2_GATE_ALPHA_PER_HEAD else full(p.log_alpha, torch.float32)
    s0 = dev(p.S0, torch.float32) if p.S0 is not None else None
    cu = dev(p.cu_seqlens, torch.int32) if p.varlen else None
    o, ST = gdn2.chunk_fwd(q, k, v, la, b, w, s0, cu)
    torch.cuda.synchronize()
    return o.reshape(-1, p.H, p.dv).cpu().numpy(), ST.cpu().numpy()


def check(p, gates, label):
    print(f'[{label}] N={p.N} tokens={p.tokens} H={p.H} dk={p.dk} dv={p.dv} {p.dtype} gates={gates}', flush=True)
    o, ST = run_gated(p, gates)
    o_ref, ST_ref = oracle_prefill(p)
    assert_close(o, o_ref, p.dtype, f'{label} o')
    assert_close(ST, ST_ref, p.dtype, f'{label} S_T')


@pytest.mark.parametrize('dt,dk,dv', [('bf16', 128, 128), ('bf16', 64, 32), ('f32', 32, 64), ('f32', 16, 16)])
@pytest.mark.parametrize('name,gates', [('kda', KDA), ('gdn', GDN), ('b', gdn2.GDN2_GATE_B_PER_HEAD),
                                        ('w', gdn2.GDN2_GATE_W_PER_HEAD), ('alpha', gdn2.GDN2_GATE_ALPHA_PER_HEAD)])
def test_gates_varlen(dt, dk, dv, name, gates):
    p = gated_batch(1100 + dk + dv, [130, 0, 64, 257, 1], 3, dk, dv, dt, gates, uniform=False)
    check(p, gates, f'{name} varlen {dt} dk={dk} dv={dv}')


@pytest.mark.parametrize('name,gates', [('kda', KDA), ('gdn', GDN)])
def test_gates_uniform_bf16(name, gates):
    p = gated_batch(1200, [300, 300], 4, 128, 128, 'bf16', gates, uniform=True, s0_std=0.0)
    check(p, gates, f'{name} uniform')


@pytest.mark.parametrize('dt', ['bf16', 'f32'])
def test_gdn_strong_scalar_decay(dt):
    """A scalar log alpha of -5 per token takes the exact diagonal-block path."""
    p = gated_batch(1300, [200, 37], 2, 128 if dt == 'bf16' else 64, 64, dt, GDN, uniform=False, s0_std=0.02)
    p.log_alpha[:] = -5.0
    check(p, GDN, f'gdn strong decay {dt}')


def test_gdn_b4_t4096_full():
    """The B=4, T=4096, H=16, d=128 bf16 workload in the Gated DeltaNet form."""
    c = gi.WORKLOADS['prefill_b4_t4096']
    p = gated_batch(c['seed'], [c['T']] * c['B'], c['H'], c['dk'], c['dv'], 'bf16', GDN, uniform=True, s0_std=0.0)
    check(p, GDN, 'gdn B=4 T=4096')


@pytest.mark.parametrize('dt,dk,dv', [('bf16', 128, 128), ('f32', 64, 32), ('bf16', 32, 16)])
@pytest.mark.parametrize('name,gates', [('kda', KDA), ('gdn', GDN), ('alpha', gdn2.GDN2_GATE_ALPHA_PER_HEAD)])
def test_decode_gates(dt, dk, dv, name, gates):
    N, H = 5, 3
    S_np = gi.decode_state(21, N, H, dk, dv, s0_std=0.3)
    S = dev(S_np, torch.float32)
    tt = tdtype(dt)
    for step in (1, 2):
        st = gi.decode_step(21, step, N, H, dk, dv, dtype=dt)
        b, w, la = st.b, st.w, st.log_alpha
        if gates & gdn2.GDN2_GATE_B_PER_HEAD:
            b = np.ascontiguousarray(np.broadcast_to(b[..., :1], b.shape))
        if gates & gdn2.GDN2_GATE_W_PER_HEAD:
            w = np.ascontiguousarray(np.broadcast_to(b[..., :1], w.shape))   # KDA: w = b = beta
        if gates & gdn2.GDN2_GATE_ALPHA_PER_HEAD:
            la = np.ascontiguousarray(np.broadcast_to(la[..., :1], la.shape))
        gb = dev(b[..., 0].copy(), tt) if gates & gdn2.GDN2_GATE_B_PER_HEAD else dev(b, tt)
        gw = dev(w[..., 0].copy(), tt) if gates & gdn2.GDN2_GATE_W_PER_HEAD else dev(w, tt)
        gla = (dev(la[..., 0].copy(), torch.float32) if gates & gdn2.GDN2_GATE_ALPHA_PER_HEAD
               else dev(la, torch.float32))
        o = gdn2.decode_step(dev(st.q, tt), dev(st.k, tt), dev(st.v, tt), gla, gb, gw, S)
        o_ref, S_np = oracle.decode_step(st.q, st.k, st.v, la, b, w, S_np)
        assert_close(o.cpu().numpy(), o_ref, 'f32', f'decode {name} {dt} step {step} o')
        assert_close(S.cpu().numpy(), S_np, 'f32', f'decode {name} {dt} step {step} S')
