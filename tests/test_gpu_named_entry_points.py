"""The two calls the C ABI is named for, gdn2_chunk_fwd and gdn2_decode_step,
called directly through ctypes with device pointers (PyTorch only allocates
the memory), against the fp64 oracle: per-channel gates, packed sequences
with ragged tails and an empty one, S0 given and absent, S_T aliasing S0."""
import ctypes

import numpy as np
import pytest

import gdn2_inputs as gi

pytestmark = pytest.mark.gpu

torch = pytest.importorskip('torch')
if not torch.cuda.is_available():
    pytest.skip('no GPU', allow_module_level=True)

import gated_delta_rule_wy_amd as gdn2  # noqa: E402
import oracle  # noqa: E402
from gpu_util import DEV, assert_close, dev, tdtype, threads  # noqa: E402

lib = gdn2.lib()
P = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    assert lib.gdn2_set_stream(ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)) == 0


@pytest.mark.parametrize('dt,dk,dv,s0,alias', [('bf16', 128, 128, True, False), ('bf16', 64, 128, False, False),
                                               ('f32', 32, 64, True, True), ('bf16', 128, 64, True, True)])
def test_chunk_fwd_direct(dt, dk, dv, s0, alias):
    lens = [300, 0, 64, 129, 1]
    p = gi.prefill(1300 + dk + dv, lens, H=3, dk=dk, dv=dv, dtype=dt, s0_std=0.05 if s0 else 0.0,
                   uniform=False)
    print(f'[gdn2_chunk_fwd] {dt} dk={dk} dv={dv} S0={s0} alias={alias}', flush=True)
    t = tdtype(dt)
    q, k, v, b, w = (dev(x, t) for x in (p.q, p.k, p.v, p.b, p.w))
    la = dev(p.log_alpha, torch.float32)
    cu = dev(p.cu_seqlens, torch.int32)
    S0 = dev(p.S0, torch.float32) if s0 else None
    o = torch.full((p.tokens, p.H, dv), float('nan'), device=DEV)
    ST = S0 if alias else torch.full((p.N, p.H, dk, dv), float('nan'), device=DEV)
    code = gdn2.GDN2_BF16 if dt == 'bf16' else gdn2.GDN2_F32
    need = lib.gdn2_chunk_fwd_workspace_bytes(1, p.tokens, p.N, p.H, dk, dv, code, 1)
    assert need > 0
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    _stream()
    st = lib.gdn2_chunk_fwd(P(q), P(k), P(v), P(la), P(b), P(w), P(S0), P(o), P(ST), P(cu),
                            1, p.tokens, p.N, p.H, dk, dv, code, gdn2.GDN2_F32, P(ws), need)
    assert st == gdn2.GDN2_OK, gdn2.status_string(st)
    torch.cuda.synchronize()
    o_ref, ST_ref = oracle.forward(p.q, p.k, p.v, p.log_alpha, p.b, p.w, p.S0 if s0 else None,
                                   cu_seqlens=p.cu_seqlens, nthreads=threads())
    assert_close(o.cpu().numpy(), o_ref, dt, 'gdn2_chunk_fwd o')
    assert_close(ST.cpu().numpy(), ST_ref, dt, 'gdn2_chunk_fwd S_T')
    # a workspace one byte short is refused before anything is launched
    st = lib.gdn2_chunk_fwd(P(q), P(k), P(v), P(la), P(b), P(w), P(S0), P(o), P(ST), P(cu),
                            1, p.tokens, p.N, p.H, dk, dv, code, gdn2.GDN2_F32, P(ws), need - 1)
    assert st == gdn2.GDN2_ERR_WORKSPACE


@pytest.mark.parametrize('dt,dk,dv', [('bf16', 128, 128), ('f32', 64, 32)])
def test_decode_step_direct(dt, dk, dv):
    N, H = 7, 5
    print(f'[gdn2_decode_step] {dt} dk={dk} dv={dv}', flush=True)
    S_np = gi.decode_state(31, N, H, dk, dv, 0.3)
    S = dev(S_np, torch.float32)
    t = tdtype(dt)
    code = gdn2.GDN2_BF16 if dt == 'bf16' else gdn2.GDN2_F32
    o = torch.empty((N, H, dv), device=DEV)
    for step in range(1, 6):
        s = gi.decode_step(31, step, N, H, dk, dv, dtype=dt)
        q, k, v, b, w = (dev(x, t) for x in (s.q, s.k, s.v, s.b, s.w))
        la = dev(s.log_alpha, torch.float32)
        _stream()
        st = lib.gdn2_decode_step(P(q), P(k), P(v), P(la), P(b), P(w), P(S), P(o), N, H, dk, dv, code,
                                  gdn2.GDN2_F32)
        assert st == gdn2.GDN2_OK, gdn2.status_string(st)
        torch.cuda.synchronize()
        o_ref, S_np = oracle.decode_step(s.q, s.k, s.v, s.log_alpha, s.b, s.w, S_np)
        assert_close(o.cpu().numpy(), o_ref, 'f32', f'gdn2_decode_step step {step} o')
    assert_close(S.cpu().numpy(), S_np, 'f32', 'gdn2_decode_step S after 5 steps')
