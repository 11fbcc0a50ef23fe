"""gdn2_chunk_fwd_noalloc (the prefill with its workspace in the library's
fixed device array, for callers that cannot allocate) against gdn2_chunk_fwd
with a caller workspace: two calls in a row, the second on a smaller input,
then a size whose workspace exceeds the array, which is refused."""
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
from gpu_util import DEV, assert_close, dev, threads  # noqa: E402

lib = gdn2.lib()
lib.gdn2_chunk_fwd_noalloc.argtypes = [ctypes.c_void_p] * 10 + [ctypes.c_int] * 8
lib.gdn2_chunk_fwd_noalloc.restype = ctypes.c_int
P = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
LIMIT = 256 << 20


def _inputs(p):
    bf = torch.bfloat16
    q, k, v, b, w = (dev(x, bf) for x in (p.q, p.k, p.v, p.b, p.w))
    return q, k, v, dev(p.log_alpha, torch.float32), b, w


def _both(p):
    """o and S_T from gdn2_chunk_fwd (caller workspace) and from the no-alloc call."""
    q, k, v, la, b, w = _inputs(p)
    S0 = dev(p.S0, torch.float32) if p.S0 is not None else None
    cu = dev(p.cu_seqlens, torch.int32)
    assert lib.gdn2_set_stream(ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)) == 0
    outs = []
    for noalloc in (False, True):
        o = torch.full((p.tokens, p.H, p.dv), float('nan'), device=DEV)
        ST = torch.full((p.N, p.H, p.dk, p.dv), float('nan'), device=DEV)
        if noalloc:
            st = lib.gdn2_chunk_fwd_noalloc(P(q), P(k), P(v), P(la), P(b), P(w), P(S0), P(o), P(ST), P(cu),
                                            1, p.tokens, p.N, p.H, p.dk, p.dv, gdn2.GDN2_BF16, gdn2.GDN2_F32)
        else:
            need = lib.gdn2_chunk_fwd_workspace_bytes(1, p.tokens, p.N, p.H, p.dk, p.dv, gdn2.GDN2_BF16, 1)
            assert 0 < need <= LIMIT
            ws = torch.empty(need, dtype=torch.uint8, device=DEV)
            st = lib.gdn2_chunk_fwd(P(q), P(k), P(v), P(la), P(b), P(w), P(S0), P(o), P(ST), P(cu),
                                    1, p.tokens, p.N, p.H, p.dk, p.dv, gdn2.GDN2_BF16, gdn2.GDN2_F32, P(ws), need)
        assert st == gdn2.GDN2_OK, gdn2.status_string(st)
        torch.cuda.synchronize()
        outs.append((o.cpu().numpy(), ST.cpu().numpy()))
    return outs


@pytest.mark.parametrize('lens,H', [([5000, 3000, 0, 4100], 16), ([300, 77], 4)])
def test_noalloc_matches_chunk_fwd(lens, H):
    # the larger call first, then a smaller one on the same (shared) array
    p = gi.prefill(1700 + H, lens, H=H, dk=128, dv=128, dtype='bf16', s0_std=0.02, uniform=False)
    print(f'[gdn2_chunk_fwd_noalloc] tokens={p.tokens} H={H}', flush=True)
    (o_ref_gpu, s_ref_gpu), (o, s) = _both(p)
    assert np.array_equal(o, o_ref_gpu) and np.array_equal(s, s_ref_gpu), 'differs from gdn2_chunk_fwd'
    o_ref, s_ref = oracle.forward(p.q, p.k, p.v, p.log_alpha, p.b, p.w, p.S0, cu_seqlens=p.cu_seqlens,
                                  nthreads=threads())
    assert_close(o, o_ref, 'bf16', 'noalloc o')
    assert_close(s, s_ref, 'bf16', 'noalloc S_T')


def test_noalloc_refuses_oversize():
    H, T = 16, 20000   # 310 MB of workspace (968 bytes per token and head)
    need = lib.gdn2_chunk_fwd_workspace_bytes(1, T, 1, H, 128, 128, gdn2.GDN2_BF16, 0)
    assert need > LIMIT
    x = torch.empty((T, H, 128), dtype=torch.bfloat16, device=DEV)
    la = torch.empty((T, H, 128), dtype=torch.float32, device=DEV)
    o = torch.empty((T, H, 128), dtype=torch.float32, device=DEV)
    st = lib.gdn2_chunk_fwd_noalloc(P(x), P(x), P(x), P(la), P(x), P(x), None, P(o), None, None,
                                    1, T, 1, H, 128, 128, gdn2.GDN2_BF16, gdn2.GDN2_F32)
    assert st == gdn2.GDN2_ERR_WORKSPACE
    # invalid arguments keep their own status
    st = lib.gdn2_chunk_fwd_noalloc(P(x), P(x), P(x), P(la), P(x), P(x), None, P(o), None, None,
                                    1, T, 1, H, 96, 128, gdn2.GDN2_BF16, gdn2.GDN2_F32)
    assert st == gdn2.GDN2_ERR_UNSUPPORTED
