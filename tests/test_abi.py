"""The C-ABI library on the CPU: it loads, exports every declared entry point,
and rejects bad arguments before touching the GPU (no compute calls here)."""
import ctypes
import os
import re

import pytest

import gated_delta_rule_wy_amd as gdn2

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, 'include', 'gdn2.h')


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r'/\*.*?\*/', '', src, flags=re.S)
    return sorted(set(re.findall(r'\b(gdn2_\w+)\s*\(', src)))


def test_header_declares_the_exports():
    assert declared_functions() == sorted(gdn2.EXPORTS)


@pytest.mark.parametrize('name', declared_functions())
def test_symbol_exported(name):
    assert hasattr(gdn2.lib(), name), name
    nm = os.popen(f'nm -D --defined-only {gdn2.LIB_PATH}').read()
    assert re.search(rf'\bT {name}\b', nm), f'{name} is not a defined dynamic symbol'


def test_status_strings():
    for s in range(5):
        assert gdn2.status_string(s).startswith('GDN2_')
    assert 'unknown' in gdn2.status_string(99)


def test_stream_is_per_thread_state():
    lib = gdn2.lib()
    assert lib.gdn2_set_stream(ctypes.c_void_p(0x1234)) == 0
    assert lib.gdn2_get_stream() == 0x1234
    import threading
    seen = []
    th = threading.Thread(target=lambda: seen.append(lib.gdn2_get_stream()))
    th.start(); th.join()
    assert seen == [None]
    lib.gdn2_set_stream(None)


WS = gdn2.lib().gdn2_chunk_fwd_workspace_bytes


def test_workspace_bytes():
    # (B, T, N, H, dk, dv, dtype, varlen)
    # layout: [chunk offsets (varlen)] [progress counters, 4 B per chain]
    # [operand blocks], each part rounded up to 256 bytes
    one = WS(1, 64, 1, 1, 128, 128, gdn2.GDN2_BF16, 0) - 256   # one (chunk, head) block
    assert one > 0 and one % 256 == 0
    assert WS(1, 65, 1, 1, 128, 128, gdn2.GDN2_BF16, 0) == 256 + 2 * one
    assert WS(4, 64, 4, 1, 128, 128, gdn2.GDN2_BF16, 0) == 256 + 4 * one
    assert WS(1, 64, 1, 3, 128, 128, gdn2.GDN2_BF16, 0) == 256 + 3 * one
    assert WS(1, 64, 1, 100, 128, 128, gdn2.GDN2_BF16, 0) == 512 + 100 * one
    # varlen reserves the chunk-offset table and one extra chunk per sequence
    assert WS(1, 64, 2, 1, 128, 128, gdn2.GDN2_BF16, 1) == 256 + 256 + 3 * one
    assert WS(1, 4096, 1, 16, 128, 128, gdn2.GDN2_F32, 0) > WS(1, 4096, 1, 16, 128, 128, gdn2.GDN2_BF16, 0)
    # invalid or unsupported sizes give 0
    assert WS(0, 64, 0, 1, 128, 128, gdn2.GDN2_BF16, 0) == 0
    assert WS(2, 64, 1, 1, 128, 128, gdn2.GDN2_BF16, 0) == 0      # N != B
    assert WS(2, 64, 2, 1, 128, 128, gdn2.GDN2_BF16, 1) == 0      # varlen needs B == 1
    assert WS(1, 64, 1, 1, 96, 128, gdn2.GDN2_BF16, 0) == 0       # dk not supported
    assert WS(1, 64, 1, 1, 16, 128, gdn2.GDN2_BF16, 0) == 0       # bf16 needs dk >= 32
    assert WS(1, 64, 1, 1, 16, 16, gdn2.GDN2_F32, 0) > 0
    assert WS(1, 64, 1, 1, 128, 128, 7, 0) == 0                   # unknown dtype


WSC = gdn2.lib().gdn2_chunk_fwd_sized_workspace_bytes


def _block_bytes(dk, bf16, C):
    """Operand block of one (chunk, head): -W and Q+ (C/16 x dk/KB fragments
    each), Khat^T (dk/16 x C/KB), the stored lower-triangle fragments of P and
    T, and gamma (dk floats); a fragment is 64 lanes x 16 bytes."""
    KB = 32 if bf16 else 16
    nrb = C // 16
    ntri = sum((16 * m + 15) // KB + 1 for m in range(nrb))
    frags = 2 * nrb * (dk // KB) + (dk // 16) * (C // KB) + 2 * ntri
    return (frags * 1024 + 4 * dk + 255) // 256 * 256


@pytest.mark.parametrize('C', [32, 64, 128])
@pytest.mark.parametrize('dt,dk', [(gdn2.GDN2_BF16, 128), (gdn2.GDN2_BF16, 32), (gdn2.GDN2_F32, 16),
                                   (gdn2.GDN2_F32, 64)])
def test_sized_workspace_bytes(C, dt, dk):
    bf = dt == gdn2.GDN2_BF16
    one = _block_bytes(dk, bf, C)
    assert WSC(1, C, 1, 1, dk, 64, dt, 0, C) == 256 + one
    assert WSC(1, C + 1, 1, 3, dk, 64, dt, 0, C) == 256 + 6 * one
    assert WSC(1, 5 * C, 2, 1, dk, 64, dt, 1, C) == 256 + 256 + 7 * one   # varlen: one extra chunk per sequence
    if C == 64:
        assert WSC(1, 4096, 1, 16, dk, 64, dt, 0, C) == WS(1, 4096, 1, 16, dk, 64, dt, 0)


def test_sized_workspace_rejects():
    assert WSC(1, 64, 1, 1, 128, 128, gdn2.GDN2_BF16, 0, 48) == 0     # chunk not 32, 64 or 128
    assert WSC(1, 64, 1, 1, 128, 128, gdn2.GDN2_BF16, 0, 256) == 0
    assert WSC(1, 64, 1, 1, 128, 128, gdn2.GDN2_F32, 0, 128) == 0     # fp32 dk=128 at C=128: LDS
    assert WSC(1, 64, 1, 1, 128, 128, gdn2.GDN2_F32, 0, 32) > 0
    assert WSC(1, 64, 1, 1, 16, 128, gdn2.GDN2_BF16, 0, 32) == 0      # bf16 needs dk >= 32


def _chunk_sized(chunk, **kw):
    P = 0x10000
    a = dict(q=P, k=P, v=P, la=P, b=P, w=P, S0=None, o=P, ST=P, cu=None, B=1, T=64, N=1, H=1,
             dk=128, dv=128, dt=gdn2.GDN2_BF16, odt=gdn2.GDN2_F32, ws=P, wsb=1 << 30)
    a.update(kw)
    vp = ctypes.c_void_p
    return gdn2.lib().gdn2_chunk_fwd_sized(*(vp(a[x]) if a[x] else None for x in
                                             ('q', 'k', 'v', 'la', 'b', 'w', 'S0', 'o', 'ST', 'cu')),
                                           a['B'], a['T'], a['N'], a['H'], a['dk'], a['dv'], a['dt'], a['odt'],
                                           chunk, vp(a['ws']) if a['ws'] else None, a['wsb'])


@pytest.mark.parametrize('chunk,kw,status', [
    (48, {}, gdn2.GDN2_ERR_INVALID),
    (0, {}, gdn2.GDN2_ERR_INVALID),
    (128, dict(dt=gdn2.GDN2_F32), gdn2.GDN2_ERR_UNSUPPORTED),
    (32, dict(q=None), gdn2.GDN2_ERR_INVALID),
    (128, dict(N=2), gdn2.GDN2_ERR_INVALID),
    (32, dict(dk=16), gdn2.GDN2_ERR_UNSUPPORTED),
    (128, dict(wsb=1024), gdn2.GDN2_ERR_WORKSPACE),
])
def test_sized_rejects(chunk, kw, status):
    assert _chunk_sized(chunk, **kw) == status


def _chunk(**kw):
    P = 0x10000   # a fake, aligned, never-dereferenced address
    a = dict(q=P, k=P, v=P, la=P, b=P, w=P, S0=None, o=P, ST=P, cu=None, B=1, T=64, N=1, H=1,
             dk=128, dv=128, dt=gdn2.GDN2_BF16, odt=gdn2.GDN2_F32, ws=P, wsb=1 << 30)
    a.update(kw)
    vp = ctypes.c_void_p
    return gdn2.lib().gdn2_chunk_fwd(*(vp(a[x]) if a[x] else None for x in
                                       ('q', 'k', 'v', 'la', 'b', 'w', 'S0', 'o', 'ST', 'cu')),
                                     a['B'], a['T'], a['N'], a['H'], a['dk'], a['dv'], a['dt'], a['odt'],
                                     vp(a['ws']) if a['ws'] else None, a['wsb'])


@pytest.mark.parametrize('kw,status', [
    (dict(q=None), gdn2.GDN2_ERR_INVALID),
    (dict(la=None), gdn2.GDN2_ERR_INVALID),
    (dict(o=None), gdn2.GDN2_ERR_INVALID),
    (dict(k=0x10004), gdn2.GDN2_ERR_INVALID),            # misaligned
    (dict(S0=0x10008), gdn2.GDN2_ERR_INVALID),
    (dict(B=0), gdn2.GDN2_ERR_INVALID),
    (dict(H=-1), gdn2.GDN2_ERR_INVALID),
    (dict(T=-5), gdn2.GDN2_ERR_INVALID),
    (dict(N=2), gdn2.GDN2_ERR_INVALID),                  # N != B without cu_seqlens
    (dict(cu=0x20000, B=2, N=2), gdn2.GDN2_ERR_INVALID), # cu_seqlens needs B == 1
    (dict(dt=5), gdn2.GDN2_ERR_INVALID),
    (dict(odt=9), gdn2.GDN2_ERR_INVALID),
    (dict(odt=gdn2.GDN2_BF16), gdn2.GDN2_ERR_UNSUPPORTED),
    (dict(dk=48), gdn2.GDN2_ERR_UNSUPPORTED),
    (dict(dv=256), gdn2.GDN2_ERR_UNSUPPORTED),
    (dict(dk=16), gdn2.GDN2_ERR_UNSUPPORTED),            # bf16 path needs dk >= 32
    (dict(ws=None), gdn2.GDN2_ERR_WORKSPACE),
    (dict(wsb=1024), gdn2.GDN2_ERR_WORKSPACE),
])
def test_chunk_fwd_rejects(kw, status):
    assert _chunk(**kw) == status


def _decode(**kw):
    P = 0x10000
    a = dict(q=P, k=P, v=P, la=P, b=P, w=P, S=P, o=P, N=4, H=2, dk=128, dv=128,
             dt=gdn2.GDN2_BF16, odt=gdn2.GDN2_F32)
    a.update(kw)
    vp = ctypes.c_void_p
    return gdn2.lib().gdn2_decode_step(*(vp(a[x]) if a[x] else None for x in
                                         ('q', 'k', 'v', 'la', 'b', 'w', 'S', 'o')),
                                       a['N'], a['H'], a['dk'], a['dv'], a['dt'], a['odt'])


@pytest.mark.parametrize('kw,status', [
    (dict(S=None), gdn2.GDN2_ERR_INVALID),
    (dict(o=None), gdn2.GDN2_ERR_INVALID),
    (dict(v=0x10002), gdn2.GDN2_ERR_INVALID),
    (dict(N=0), gdn2.GDN2_ERR_INVALID),
    (dict(dk=100), gdn2.GDN2_ERR_UNSUPPORTED),
    (dict(dt=3), gdn2.GDN2_ERR_INVALID),
    (dict(odt=gdn2.GDN2_BF16), gdn2.GDN2_ERR_UNSUPPORTED),
])
def test_decode_rejects(kw, status):
    assert _decode(**kw) == status


@pytest.mark.parametrize('gates', [8, 16, -1])
def test_gate_layout_rejects_unknown_bits(gates):
    P = 0x10000
    vp = ctypes.c_void_p
    lib = gdn2.lib()
    st = lib.gdn2_chunk_fwd_gates(vp(P), vp(P), vp(P), vp(P), vp(P), vp(P), gates, None, vp(P), vp(P), None,
                                  1, 64, 1, 1, 128, 128, gdn2.GDN2_BF16, gdn2.GDN2_F32, vp(P), 1 << 30)
    assert st == gdn2.GDN2_ERR_INVALID
    st = lib.gdn2_decode_step_gates(vp(P), vp(P), vp(P), vp(P), vp(P), vp(P), gates, vp(P), vp(P),
                                    4, 2, 128, 128, gdn2.GDN2_BF16, gdn2.GDN2_F32)
    assert st == gdn2.GDN2_ERR_INVALID


def test_gate_layout_valid_bits_pass_validation():
    """Known layouts pass host validation (a bad dk then decides the status, so nothing launches)."""
    P = 0x10000
    vp = ctypes.c_void_p
    lib = gdn2.lib()
    for gates in range(8):
        st = lib.gdn2_chunk_fwd_gates(vp(P), vp(P), vp(P), vp(P), vp(P), vp(P), gates, None, vp(P), vp(P),
                                      None, 1, 64, 1, 1, 48, 128, gdn2.GDN2_BF16, gdn2.GDN2_F32, vp(P), 1 << 30)
        assert st == gdn2.GDN2_ERR_UNSUPPORTED


def test_python_binding_validates_before_calling():
    import torch
    x = torch.zeros(1, 64, 1, 128, dtype=torch.bfloat16)
    la = torch.zeros(1, 64, 1, 128)
    with pytest.raises(TypeError):
        gdn2.chunk_fwd(x, x, x, la.to(torch.bfloat16), x, x)
    with pytest.raises(ValueError):
        gdn2.chunk_fwd(x, x[:, :32], x, la, x, x)
    with pytest.raises(TypeError):
        gdn2.chunk_fwd(x.half(), x.half(), x.half(), la, x.half(), x.half())


def _conv(**kw):
    P = 0x10000
    c = gdn2.ShortConv(weight_q=P, weight_k=P, weight_v=P)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


@pytest.mark.parametrize('kw,status', [
    (None, gdn2.GDN2_ERR_INVALID),                                   # no struct
    (dict(weight_k=None), gdn2.GDN2_ERR_INVALID),                    # taps required
    (dict(weight_v=0x10004), gdn2.GDN2_ERR_INVALID),                 # misaligned
    (dict(bias_q=0x10008), gdn2.GDN2_ERR_INVALID),
    (dict(state_in_q=0x20000), gdn2.GDN2_ERR_INVALID),               # history in: all or none
    (dict(state_out_q=0x20000, state_out_k=0x20000), gdn2.GDN2_ERR_INVALID),
    (dict(), gdn2.GDN2_ERR_WORKSPACE),                               # valid: the small workspace decides
    (dict(bias_q=0x30000, bias_v=0x30000), gdn2.GDN2_ERR_WORKSPACE),
    (dict(state_in_q=0x20000, state_in_k=0x20000, state_in_v=0x20000,
          state_out_q=0x20000, state_out_k=0x20000, state_out_v=0x20000), gdn2.GDN2_ERR_WORKSPACE),
])
def test_prologue_conv_validation(kw, status):
    """The convolution struct is checked on the host before anything launches."""
    P = 0x10000
    vp = ctypes.c_void_p
    conv = None if kw is None else ctypes.byref(_conv(**kw))
    st = gdn2.lib().gdn2_chunk_fwd_prologue(vp(P), vp(P), vp(P), vp(P), vp(P), vp(P), conv, None, vp(P), vp(P),
                                            None, 1, 64, 1, 1, 128, 128, gdn2.GDN2_BF16, gdn2.GDN2_F32, vp(P), 1024)
    assert st == status
    if status == gdn2.GDN2_ERR_INVALID:
        st = gdn2.lib().gdn2_decode_step_prologue(vp(P), vp(P), vp(P), vp(P), vp(P), vp(P), conv, vp(P), vp(P),
                                                  4, 2, 128, 128, gdn2.GDN2_BF16, gdn2.GDN2_F32)
        assert st == status


def test_prologue_binding_validates_before_calling():
    import torch
    x = torch.zeros(1, 64, 1, 128, dtype=torch.bfloat16)
    la = torch.zeros(1, 64, 1, 128)
    wt = tuple(torch.zeros(128, 4) for _ in range(3))
    with pytest.raises(ValueError):            # taps of the wrong shape
        gdn2.chunk_fwd_prologue(x, x, x, la, x, x, (wt[0], wt[1], torch.zeros(128, 3)))
    with pytest.raises(ValueError):            # not a triple
        gdn2.chunk_fwd_prologue(x, x, x, la, x, x, wt[:2])
    with pytest.raises(TypeError):             # history in the wrong dtype
        gdn2.chunk_fwd_prologue(x, x, x, la, x, x, wt,
                                conv_state=tuple(torch.zeros(1, 1, 3, 128) for _ in range(3)))


# ---- the training pair (gdn2_chunk_fwd_keep / gdn2_chunk_bwd_kept): every
# check runs before a launch, so fake aligned addresses never reach a kernel

def _keep(**kw):
    P = 0x10000
    a = dict(q=P, k=P, v=P, la=P, b=P, w=P, S0=None, o=P, ST=P, cu=None, B=1, T=64, N=1, H=1,
             dk=128, dv=128, dt=gdn2.GDN2_BF16, odt=gdn2.GDN2_F32, ws=P, wsb=1 << 30)
    a.update(kw)
    vp = ctypes.c_void_p
    return gdn2.lib().gdn2_chunk_fwd_keep(*(vp(a[x]) if a[x] else None for x in
                                            ('q', 'k', 'v', 'la', 'b', 'w', 'S0', 'o', 'ST', 'cu')),
                                          a['B'], a['T'], a['N'], a['H'], a['dk'], a['dv'], a['dt'], a['odt'],
                                          vp(a['ws']) if a['ws'] else None, a['wsb'])


def _kept(**kw):
    P = 0x10000
    a = dict(q=P, k=P, v=P, la=P, b=P, w=P, S0=None, dO=P, dST=None, cu=None, B=1, T=64, N=1, H=1,
             dk=128, dv=128, dt=gdn2.GDN2_BF16, dq=P, dk_=P, dv_=P, dla=P, db=P, dw=P, dS0=None,
             ws=P, wsb=1 << 30)
    a.update(kw)
    vp = ctypes.c_void_p
    ptr = lambda x: vp(a[x]) if a[x] else None
    return gdn2.lib().gdn2_chunk_bwd_kept(*(ptr(x) for x in ('q', 'k', 'v', 'la', 'b', 'w', 'S0', 'dO', 'dST', 'cu')),
                                          a['B'], a['T'], a['N'], a['H'], a['dk'], a['dv'], a['dt'],
                                          *(ptr(x) for x in ('dq', 'dk_', 'dv_', 'dla', 'db', 'dw', 'dS0', 'ws')),
                                          a['wsb'])


BWS = gdn2.lib().gdn2_chunk_bwd_workspace_bytes


@pytest.mark.parametrize('kw,status', [
    (dict(q=None), gdn2.GDN2_ERR_INVALID),
    (dict(o=None), gdn2.GDN2_ERR_INVALID),
    (dict(w=0x10004), gdn2.GDN2_ERR_INVALID),
    (dict(ST=0x10008), gdn2.GDN2_ERR_INVALID),
    (dict(N=2), gdn2.GDN2_ERR_INVALID),
    (dict(odt=gdn2.GDN2_BF16), gdn2.GDN2_ERR_UNSUPPORTED),
    (dict(odt=7), gdn2.GDN2_ERR_INVALID),
    (dict(dk=48), gdn2.GDN2_ERR_UNSUPPORTED),
    (dict(ws=None), gdn2.GDN2_ERR_WORKSPACE),
    # the forward's own workspace is too small: the backward's is needed
    (dict(wsb=WS(1, 64, 1, 1, 128, 128, gdn2.GDN2_BF16, 0)), gdn2.GDN2_ERR_WORKSPACE),
    (dict(wsb=BWS(1, 64, 1, 1, 128, 128, gdn2.GDN2_BF16, 0) - 1), gdn2.GDN2_ERR_WORKSPACE),
])
def test_chunk_fwd_keep_rejects(kw, status):
    assert _keep(**kw) == status


@pytest.mark.parametrize('kw,status', [
    (dict(dO=None), gdn2.GDN2_ERR_INVALID),
    (dict(dla=None), gdn2.GDN2_ERR_INVALID),
    (dict(dS0=0x10004), gdn2.GDN2_ERR_INVALID),
    (dict(T=-1), gdn2.GDN2_ERR_INVALID),
    (dict(dv=100), gdn2.GDN2_ERR_UNSUPPORTED),
    (dict(ws=None), gdn2.GDN2_ERR_WORKSPACE),
    (dict(wsb=BWS(1, 64, 1, 1, 128, 128, gdn2.GDN2_BF16, 0) - 1), gdn2.GDN2_ERR_WORKSPACE),
])
def test_chunk_bwd_kept_rejects(kw, status):
    assert _kept(**kw) == status


def test_kept_binding_needs_the_workspace():
    torch = pytest.importorskip('torch')
    x = torch.zeros(1, 64, 1, 128, dtype=torch.bfloat16)
    la = torch.zeros(1, 64, 1, 128)
    with pytest.raises(ValueError, match='workspace'):
        gdn2.chunk_bwd_kept(x, x, x, la, x, x, None, la, workspace=torch.zeros(16, dtype=torch.uint8))
