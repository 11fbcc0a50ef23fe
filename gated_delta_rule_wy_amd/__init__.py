"""Gated DeltaNet-2 token mixer for MI355X (gfx950): Python binding of libgdn2.

A thin ctypes layer over the C ABI in ``include/gdn2.h``: it checks tensor
shapes, dtypes and devices, allocates outputs and workspace with PyTorch, sets
the library's stream to PyTorch's current stream and calls the library. Every
step of the computation runs in the HIP kernels; there is no other code path,
and importing this package fails if the library has not been built.

Recurrence (snilld.dk, "Hvad Gated DeltaNet-2 ændrer", update equation), per
sequence and head, state S in R^{dk x dv}:
    S_t = (I - k_t (b_t * k_t)^T) Diag(exp(log_alpha_t)) S_{t-1} + k_t (w_t * v_t)^T
    o_t = S_t^T q_t
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, 'libgdn2.so')

GDN2_OK, GDN2_ERR_INVALID, GDN2_ERR_UNSUPPORTED, GDN2_ERR_WORKSPACE, GDN2_ERR_HIP = range(5)
GDN2_F32, GDN2_BF16 = 0, 1
GDN2_GATES_PER_CHANNEL, GDN2_GATE_B_PER_HEAD, GDN2_GATE_W_PER_HEAD, GDN2_GATE_ALPHA_PER_HEAD = 0, 1, 2, 4
CHUNK = 64

EXPORTS = ('gdn2_set_stream', 'gdn2_get_stream', 'gdn2_status_string',
           'gdn2_chunk_fwd_workspace_bytes', 'gdn2_chunk_fwd', 'gdn2_chunk_fwd_noalloc', 'gdn2_chunk_fwd_gates',
           'gdn2_chunk_fwd_sized_workspace_bytes', 'gdn2_chunk_fwd_sized',
           'gdn2_decode_step', 'gdn2_decode_step_gates',
           'gdn2_chunk_fwd_prologue', 'gdn2_decode_step_prologue',
           'gdn2_chunk_bwd_workspace_bytes', 'gdn2_chunk_bwd', 'gdn2_chunk_fwd_keep', 'gdn2_chunk_bwd_kept',
           'gdn2_profile_begin', 'gdn2_profile_end', 'gdn2_profile_kernel')


class ShortConv(ctypes.Structure):
    """gdn2_short_conv: taps, biases and history of the three short convolutions."""
    _fields_ = [(n, ctypes.c_void_p) for n in (
        'weight_q', 'weight_k', 'weight_v', 'bias_q', 'bias_k', 'bias_v',
        'state_in_q', 'state_in_k', 'state_in_v', 'state_out_q', 'state_out_k', 'state_out_v')]


class Gdn2Error(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f'{where}: {status_string(status)}')
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f'{LIB_PATH} is missing: build it first (python -c "import __graft_entry__ as g; g.build()")')
    lib = ctypes.CDLL(LIB_PATH)
    vp, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.gdn2_set_stream.argtypes = [vp]
    lib.gdn2_set_stream.restype = i
    lib.gdn2_get_stream.argtypes = []
    lib.gdn2_get_stream.restype = vp
    lib.gdn2_status_string.argtypes = [i]
    lib.gdn2_status_string.restype = ctypes.c_char_p
    lib.gdn2_chunk_fwd_workspace_bytes.argtypes = [i] * 8
    lib.gdn2_chunk_fwd_workspace_bytes.restype = sz
    lib.gdn2_chunk_fwd.argtypes = [vp] * 10 + [i] * 8 + [vp, sz]
    lib.gdn2_chunk_fwd.restype = i
    lib.gdn2_chunk_fwd_noalloc.argtypes = [vp] * 10 + [i] * 8
    lib.gdn2_chunk_fwd_noalloc.restype = i
    lib.gdn2_chunk_fwd_gates.argtypes = [vp] * 6 + [i] + [vp] * 4 + [i] * 8 + [vp, sz]
    lib.gdn2_chunk_fwd_gates.restype = i
    lib.gdn2_chunk_fwd_sized_workspace_bytes.argtypes = [i] * 9
    lib.gdn2_chunk_fwd_sized_workspace_bytes.restype = sz
    lib.gdn2_chunk_fwd_sized.argtypes = [vp] * 10 + [i] * 9 + [vp, sz]
    lib.gdn2_chunk_fwd_sized.restype = i
    lib.gdn2_decode_step.argtypes = [vp] * 8 + [i] * 6
    lib.gdn2_decode_step.restype = i
    lib.gdn2_decode_step_gates.argtypes = [vp] * 6 + [i] + [vp] * 2 + [i] * 6
    lib.gdn2_decode_step_gates.restype = i
    pc = ctypes.POINTER(ShortConv)
    lib.gdn2_chunk_fwd_prologue.argtypes = [vp] * 6 + [pc] + [vp] * 4 + [i] * 8 + [vp, sz]
    lib.gdn2_chunk_fwd_prologue.restype = i
    lib.gdn2_decode_step_prologue.argtypes = [vp] * 6 + [pc] + [vp] * 2 + [i] * 6
    lib.gdn2_decode_step_prologue.restype = i
    lib.gdn2_chunk_bwd_workspace_bytes.argtypes = [i] * 8
    lib.gdn2_chunk_bwd_workspace_bytes.restype = sz
    lib.gdn2_chunk_bwd.argtypes = [vp] * 10 + [i] * 7 + [vp] * 7 + [vp, sz]
    lib.gdn2_chunk_bwd.restype = i
    lib.gdn2_chunk_fwd_keep.argtypes = [vp] * 10 + [i] * 8 + [vp, sz]
    lib.gdn2_chunk_fwd_keep.restype = i
    lib.gdn2_chunk_bwd_kept.argtypes = [vp] * 10 + [i] * 7 + [vp] * 7 + [vp, sz]
    lib.gdn2_chunk_bwd_kept.restype = i
    lib.gdn2_profile_begin.argtypes = [i]
    lib.gdn2_profile_begin.restype = i
    lib.gdn2_profile_end.argtypes = []
    lib.gdn2_profile_end.restype = i
    lib.gdn2_profile_kernel.argtypes = [i, ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(ctypes.c_int),
                                        ctypes.POINTER(ctypes.c_double)]
    lib.gdn2_profile_kernel.restype = i
    return lib


_lib = _load()


def lib() -> ctypes.CDLL:
    return _lib


def status_string(status: int) -> str:
    return _lib.gdn2_status_string(int(status)).decode()


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return GDN2_BF16
    if t.dtype == torch.float32:
        return GDN2_F32
    raise TypeError(f'unsupported input dtype {t.dtype} (bfloat16 or float32)')


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(t: torch.Tensor, name: str, shape, dtype, device):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f'{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}')
    if t.dtype != dtype:
        raise TypeError(f'{name}: expected {dtype}, got {t.dtype}')
    if t.device != device:
        raise ValueError(f'{name}: expected device {device}, got {t.device}')
    if not t.is_contiguous():
        raise ValueError(f'{name}: must be contiguous')


def set_stream(stream: Optional[torch.cuda.Stream] = None) -> None:
    """Point the library at ``stream`` (default: PyTorch's current stream)."""
    s = torch.cuda.current_stream() if stream is None else stream
    _lib.gdn2_set_stream(ctypes.c_void_p(s.cuda_stream))


def workspace_bytes(B: int, T: int, N: int, H: int, dk: int, dv: int, dtype: torch.dtype,
                    varlen: bool, chunk: int = CHUNK) -> int:
    code = GDN2_BF16 if dtype == torch.bfloat16 else GDN2_F32
    return int(_lib.gdn2_chunk_fwd_sized_workspace_bytes(B, T, N, H, dk, dv, code, int(varlen), int(chunk)))


def profile_begin(max_calls: int) -> None:
    """Time each kernel of this thread's next ``max_calls`` library calls with HIP events."""
    st = _lib.gdn2_profile_begin(int(max_calls))
    if st != GDN2_OK:
        raise Gdn2Error(st, 'gdn2_profile_begin')


def profile_end() -> dict:
    """Stop recording; return {kernel name: (launches, total ms)} for the recorded calls."""
    _lib.gdn2_profile_end()
    out = {}
    idx = 0
    while True:
        name, n, ms = ctypes.c_char_p(), ctypes.c_int(), ctypes.c_double()
        st = _lib.gdn2_profile_kernel(idx, ctypes.byref(name), ctypes.byref(n), ctypes.byref(ms))
        if st == GDN2_ERR_INVALID:
            break
        if st != GDN2_OK:
            raise Gdn2Error(st, 'gdn2_profile_kernel')
        out[name.value.decode()] = (n.value, ms.value)
        idx += 1
    return out


def _gate_layout(lead, H, dk, dv, b, w, log_alpha, dt, dev) -> int:
    """Gate layout bits from the gate shapes: a gate without the channel axis
    ([..., H]) holds one value per token-head (KDA / Gated DeltaNet forms)."""
    gates = 0
    for name, t, d, bit, tdt in (('b', b, dk, GDN2_GATE_B_PER_HEAD, dt), ('w', w, dv, GDN2_GATE_W_PER_HEAD, dt),
                                 ('log_alpha', log_alpha, dk, GDN2_GATE_ALPHA_PER_HEAD, torch.float32)):
        if t.dim() == len(lead) + 1:
            _check(t, name, (*lead, H), tdt, dev)
            gates |= bit
        else:
            _check(t, name, (*lead, H, d), tdt, dev)
    return gates


def chunk_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, log_alpha: torch.Tensor,
              b: torch.Tensor, w: torch.Tensor, S0: Optional[torch.Tensor] = None,
              cu_seqlens: Optional[torch.Tensor] = None, *, out: Optional[torch.Tensor] = None,
              final_state: Optional[torch.Tensor] = None, output_final_state: bool = True,
              workspace: Optional[torch.Tensor] = None,
              chunk: int = CHUNK) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Chunkwise prefill. q, k, b: [B, T, H, dk]; v, w: [B, T, H, dv] (bf16 or
    fp32); log_alpha: [B, T, H, dk] fp32. With ``cu_seqlens`` (int32 [N+1] on
    the device) B must be 1 and the sequences are packed along T. S0: [N, H,
    dk, dv] fp32 or None (zeros). Returns (o [B, T, H, dv] fp32, S_T [N, H, dk,
    dv] fp32 or None). b, w and log_alpha may instead be [B, T, H], one gate
    per token-head (KDA: b = w = beta; Gated DeltaNet: also a scalar decay).
    ``chunk``: tokens per chunk, 64, or 32 / 128 (gdn2_chunk_fwd_sized,
    per-channel gates only)."""
    if q.dim() != 4:
        raise ValueError('q must be [B, T, H, dk]')
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    code = _dtype_code(q)
    for name, t, d in (('q', q, dk), ('k', k, dk), ('v', v, dv)):
        _check(t, name, (B, T, H, d), dt, dev)
    gates = _gate_layout((B, T), H, dk, dv, b, w, log_alpha, dt, dev)
    if cu_seqlens is not None:
        if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or cu_seqlens.device != dev:
            raise ValueError('cu_seqlens must be a 1-D int32 tensor on the same device')
        if not cu_seqlens.is_contiguous():
            raise ValueError('cu_seqlens must be contiguous')
        N = cu_seqlens.numel() - 1
    else:
        N = B
    if S0 is not None:
        _check(S0, 'S0', (N, H, dk, dv), torch.float32, dev)
    if out is None:
        out = torch.empty((B, T, H, dv), dtype=torch.float32, device=dev)
    else:
        _check(out, 'out', (B, T, H, dv), torch.float32, dev)
    ST = None
    if final_state is not None:
        _check(final_state, 'final_state', (N, H, dk, dv), torch.float32, dev)
        ST = final_state
    elif output_final_state:
        ST = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
    varlen = cu_seqlens is not None
    if chunk != CHUNK and gates != GDN2_GATES_PER_CHANNEL:
        raise ValueError(f'chunk = {chunk} takes per-channel gates only')
    need = _lib.gdn2_chunk_fwd_sized_workspace_bytes(B, T, N, H, dk, dv, code, int(varlen), int(chunk))
    if need == 0:
        raise Gdn2Error(GDN2_ERR_UNSUPPORTED, 'gdn2_chunk_fwd_sized_workspace_bytes')
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    set_stream()
    wsb = workspace.numel() * workspace.element_size()
    if chunk == CHUNK and gates == GDN2_GATES_PER_CHANNEL:
        st = _lib.gdn2_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(b), _ptr(w),
                                 _ptr(S0), _ptr(out), _ptr(ST), _ptr(cu_seqlens),
                                 B, T, N, H, dk, dv, code, GDN2_F32, _ptr(workspace), wsb)
        where = 'gdn2_chunk_fwd'
    elif chunk == CHUNK:
        st = _lib.gdn2_chunk_fwd_gates(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(b), _ptr(w), gates,
                                       _ptr(S0), _ptr(out), _ptr(ST), _ptr(cu_seqlens),
                                       B, T, N, H, dk, dv, code, GDN2_F32, _ptr(workspace), wsb)
        where = 'gdn2_chunk_fwd_gates'
    else:
        st = _lib.gdn2_chunk_fwd_sized(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(b), _ptr(w),
                                       _ptr(S0), _ptr(out), _ptr(ST), _ptr(cu_seqlens),
                                       B, T, N, H, dk, dv, code, GDN2_F32, int(chunk), _ptr(workspace), wsb)
        where = 'gdn2_chunk_fwd_sized'
    if st != GDN2_OK:
        raise Gdn2Error(st, where)
    return out, ST


def decode_step(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, log_alpha: torch.Tensor,
                b: torch.Tensor, w: torch.Tensor, S: torch.Tensor, *,
                out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One token per sequence. q, k, b: [N, H, dk]; v, w: [N, H, dv]; log_alpha
    [N, H, dk] fp32; S: [N, H, dk, dv] fp32, updated in place. Returns o [N, H, dv] fp32.
    b, w and log_alpha may instead be [N, H] (one gate per sequence-head)."""
    if q.dim() != 3:
        raise ValueError('q must be [N, H, dk]')
    N, H, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    code = _dtype_code(q)
    for name, t, d in (('q', q, dk), ('k', k, dk), ('v', v, dv)):
        _check(t, name, (N, H, d), dt, dev)
    gates = _gate_layout((N,), H, dk, dv, b, w, log_alpha, dt, dev)
    _check(S, 'S', (N, H, dk, dv), torch.float32, dev)
    if out is None:
        out = torch.empty((N, H, dv), dtype=torch.float32, device=dev)
    else:
        _check(out, 'out', (N, H, dv), torch.float32, dev)
    set_stream()
    if gates == GDN2_GATES_PER_CHANNEL:
        st = _lib.gdn2_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(b), _ptr(w),
                                   _ptr(S), _ptr(out), N, H, dk, dv, code, GDN2_F32)
        where = 'gdn2_decode_step'
    else:
        st = _lib.gdn2_decode_step_gates(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(b), _ptr(w), gates,
                                         _ptr(S), _ptr(out), N, H, dk, dv, code, GDN2_F32)
        where = 'gdn2_decode_step_gates'
    if st != GDN2_OK:
        raise Gdn2Error(st, where)
    return out


def _short_conv(H, dk, dv, dev, dt, lead_n, weight, bias, state_in, state_out) -> ShortConv:
    """Marshal (q, k, v) triples of taps, biases and histories into a ShortConv."""
    dims = (dk, dk, dv)
    if weight is None or len(weight) != 3:
        raise ValueError('conv_weight must be a (q, k, v) triple of [H*d, 4] float32 tensors')
    sc = ShortConv()
    for n, t, d in zip('qkv', weight, dims):
        _check(t, f'conv_weight[{n}]', (H * d, 4), torch.float32, dev)
        setattr(sc, f'weight_{n}', t.data_ptr())
    if bias is not None:
        for n, t, d in zip('qkv', bias, dims):
            if t is not None:
                _check(t, f'conv_bias[{n}]', (H * d,), torch.float32, dev)
                setattr(sc, f'bias_{n}', t.data_ptr())
    for label, trip in (('in', state_in), ('out', state_out)):
        if trip is None:
            continue
        for n, t, d in zip('qkv', trip, dims):
            _check(t, f'conv_state_{label}[{n}]', (lead_n, H, 3, d), dt, dev)
            setattr(sc, f'state_{label}_{n}', t.data_ptr())
    return sc


def chunk_fwd_prologue(q_raw: torch.Tensor, k_raw: torch.Tensor, v_raw: torch.Tensor, log_alpha: torch.Tensor,
                       b_logit: torch.Tensor, w_logit: torch.Tensor, conv_weight, conv_bias=None,
                       S0: Optional[torch.Tensor] = None, cu_seqlens: Optional[torch.Tensor] = None, *,
                       conv_state=None, conv_state_out=None, output_conv_state: bool = True,
                       out: Optional[torch.Tensor] = None, final_state: Optional[torch.Tensor] = None,
                       output_final_state: bool = True, workspace: Optional[torch.Tensor] = None):
    """Prefill on the projections' outputs, with the prologue fused in:
    q = L2Norm(ShortConv(q_raw)), k = L2Norm(ShortConv(k_raw)), v = ShortConv(v_raw),
    b = sigmoid(b_logit), w = sigmoid(w_logit).

    Shapes as in ``chunk_fwd`` (gates per channel). conv_weight: (q, k, v) taps
    [H*dk, 4], [H*dk, 4], [H*dv, 4] float32, tap 3 on the current token;
    conv_bias: such a triple of [H*d] (entries may be None) or None.
    conv_state: (q, k, v) histories [N, H, 3, d] in the input dtype (the
    three raw inputs before each sequence, oldest first) or None for zeros.
    conv_state_out: tensors to receive the new histories (may be conv_state
    itself); allocated when None and ``output_conv_state``.
    Returns (o, S_T or None, conv_state_out triple or None).
    """
    if q_raw.dim() != 4:
        raise ValueError('q_raw must be [B, T, H, dk]')
    B, T, H, dk = q_raw.shape
    dv = v_raw.shape[-1]
    dev, dt = q_raw.device, q_raw.dtype
    code = _dtype_code(q_raw)
    for name, t, d in (('q_raw', q_raw, dk), ('k_raw', k_raw, dk), ('v_raw', v_raw, dv),
                       ('b_logit', b_logit, dk), ('w_logit', w_logit, dv)):
        _check(t, name, (B, T, H, d), dt, dev)
    _check(log_alpha, 'log_alpha', (B, T, H, dk), torch.float32, dev)
    if cu_seqlens is not None:
        if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or cu_seqlens.device != dev:
            raise ValueError('cu_seqlens must be a 1-D int32 tensor on the same device')
        if not cu_seqlens.is_contiguous():
            raise ValueError('cu_seqlens must be contiguous')
        N = cu_seqlens.numel() - 1
    else:
        N = B
    if S0 is not None:
        _check(S0, 'S0', (N, H, dk, dv), torch.float32, dev)
    if out is None:
        out = torch.empty((B, T, H, dv), dtype=torch.float32, device=dev)
    else:
        _check(out, 'out', (B, T, H, dv), torch.float32, dev)
    ST = None
    if final_state is not None:
        _check(final_state, 'final_state', (N, H, dk, dv), torch.float32, dev)
        ST = final_state
    elif output_final_state:
        ST = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
    if conv_state_out is None and output_conv_state:
        conv_state_out = tuple(torch.empty((N, H, 3, d), dtype=dt, device=dev) for d in (dk, dk, dv))
    sc = _short_conv(H, dk, dv, dev, dt, N, conv_weight, conv_bias, conv_state, conv_state_out)
    varlen = cu_seqlens is not None
    need = _lib.gdn2_chunk_fwd_workspace_bytes(B, T, N, H, dk, dv, code, int(varlen))
    if need == 0:
        raise Gdn2Error(GDN2_ERR_UNSUPPORTED, 'gdn2_chunk_fwd_workspace_bytes')
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    set_stream()
    st = _lib.gdn2_chunk_fwd_prologue(_ptr(q_raw), _ptr(k_raw), _ptr(v_raw), _ptr(log_alpha), _ptr(b_logit),
                                      _ptr(w_logit), ctypes.byref(sc), _ptr(S0), _ptr(out), _ptr(ST),
                                      _ptr(cu_seqlens), B, T, N, H, dk, dv, code, GDN2_F32, _ptr(workspace),
                                      workspace.numel() * workspace.element_size())
    if st != GDN2_OK:
        raise Gdn2Error(st, 'gdn2_chunk_fwd_prologue')
    return out, ST, conv_state_out


def decode_step_prologue(q_raw: torch.Tensor, k_raw: torch.Tensor, v_raw: torch.Tensor, log_alpha: torch.Tensor,
                         b_logit: torch.Tensor, w_logit: torch.Tensor, S: torch.Tensor, conv_weight,
                         conv_bias=None, conv_state=None, *, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One token per sequence on raw inputs ([N, H, d]), prologue fused in.
    S [N, H, dk, dv] float32 and the conv_state histories ((q, k, v) triple
    of [N, H, 3, d], or None for zeros) are updated in place. Returns o."""
    if q_raw.dim() != 3:
        raise ValueError('q_raw must be [N, H, dk]')
    N, H, dk = q_raw.shape
    dv = v_raw.shape[-1]
    dev, dt = q_raw.device, q_raw.dtype
    code = _dtype_code(q_raw)
    for name, t, d in (('q_raw', q_raw, dk), ('k_raw', k_raw, dk), ('v_raw', v_raw, dv),
                       ('b_logit', b_logit, dk), ('w_logit', w_logit, dv)):
        _check(t, name, (N, H, d), dt, dev)
    _check(log_alpha, 'log_alpha', (N, H, dk), torch.float32, dev)
    _check(S, 'S', (N, H, dk, dv), torch.float32, dev)
    if out is None:
        out = torch.empty((N, H, dv), dtype=torch.float32, device=dev)
    else:
        _check(out, 'out', (N, H, dv), torch.float32, dev)
    sc = _short_conv(H, dk, dv, dev, dt, N, conv_weight, conv_bias, conv_state, conv_state)
    set_stream()
    st = _lib.gdn2_decode_step_prologue(_ptr(q_raw), _ptr(k_raw), _ptr(v_raw), _ptr(log_alpha), _ptr(b_logit),
                                        _ptr(w_logit), ctypes.byref(sc), _ptr(S), _ptr(out), N, H, dk, dv, code,
                                        GDN2_F32)
    if st != GDN2_OK:
        raise Gdn2Error(st, 'gdn2_decode_step_prologue')
    return out


def _seq_count(cu_seqlens, B, dev):
    if cu_seqlens is None:
        return B
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or cu_seqlens.device != dev:
        raise ValueError('cu_seqlens must be a 1-D int32 tensor on the same device')
    if not cu_seqlens.is_contiguous():
        raise ValueError('cu_seqlens must be contiguous')
    return cu_seqlens.numel() - 1


def bwd_workspace_bytes(B: int, T: int, N: int, H: int, dk: int, dv: int, dtype: torch.dtype, varlen: bool) -> int:
    """Device workspace of chunk_bwd, chunk_fwd_keep and chunk_bwd_kept."""
    code = GDN2_BF16 if dtype == torch.bfloat16 else GDN2_F32
    need = _lib.gdn2_chunk_bwd_workspace_bytes(B, T, N, H, dk, dv, code, int(varlen))
    if need == 0:
        raise Gdn2Error(GDN2_ERR_UNSUPPORTED, 'gdn2_chunk_bwd_workspace_bytes')
    return need


def _bwd(fn: str, q, k, v, log_alpha, b, w, S0, dO, dST, cu_seqlens, workspace, need_workspace) -> dict:
    if q.dim() != 4:
        raise ValueError('q must be [B, T, H, dk]')
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    code = _dtype_code(q)
    for name, t, d in (('q', q, dk), ('k', k, dk), ('v', v, dv), ('b', b, dk), ('w', w, dv)):
        _check(t, name, (B, T, H, d), dt, dev)
    _check(log_alpha, 'log_alpha', (B, T, H, dk), torch.float32, dev)
    _check(dO, 'dO', (B, T, H, dv), torch.float32, dev)
    N = _seq_count(cu_seqlens, B, dev)
    for name, t in (('S0', S0), ('dST', dST)):
        if t is not None:
            _check(t, name, (N, H, dk, dv), torch.float32, dev)
    g = {name: torch.empty((B, T, H, d), dtype=torch.float32, device=dev)
         for name, d in (('q', dk), ('k', dk), ('v', dv), ('log_alpha', dk), ('b', dk), ('w', dv))}
    g['S0'] = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
    need = bwd_workspace_bytes(B, T, N, H, dk, dv, dt, cu_seqlens is not None)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        if need_workspace:
            raise ValueError(f'{fn}: pass the workspace of the matching chunk_fwd_keep ({need} bytes)')
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    set_stream()
    st = getattr(_lib, fn)(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(b), _ptr(w), _ptr(S0), _ptr(dO),
                           _ptr(dST), _ptr(cu_seqlens), B, T, N, H, dk, dv, code,
                           _ptr(g['q']), _ptr(g['k']), _ptr(g['v']), _ptr(g['log_alpha']), _ptr(g['b']),
                           _ptr(g['w']), _ptr(g['S0']), _ptr(workspace),
                           workspace.numel() * workspace.element_size())
    if st != GDN2_OK:
        raise Gdn2Error(st, fn)
    return g


def chunk_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, log_alpha: torch.Tensor,
              b: torch.Tensor, w: torch.Tensor, S0: Optional[torch.Tensor], dO: torch.Tensor,
              dST: Optional[torch.Tensor] = None, cu_seqlens: Optional[torch.Tensor] = None, *,
              workspace: Optional[torch.Tensor] = None) -> dict:
    """Gradients of a loss through ``chunk_fwd`` (per-channel gates): given
    dO = dL/do [B, T, H, dv] float32 and dST = dL/dS_T [N, H, dk, dv] (or
    None), returns float32 tensors {'q', 'k', 'v', 'log_alpha', 'b', 'w'}
    shaped like those inputs and 'S0' [N, H, dk, dv]."""
    return _bwd('gdn2_chunk_bwd', q, k, v, log_alpha, b, w, S0, dO, dST, cu_seqlens, workspace, False)


def chunk_fwd_keep(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, log_alpha: torch.Tensor,
                   b: torch.Tensor, w: torch.Tensor, S0: Optional[torch.Tensor] = None,
                   cu_seqlens: Optional[torch.Tensor] = None, *,
                   workspace: Optional[torch.Tensor] = None):
    """The training forward (gdn2_chunk_fwd_keep): ``chunk_fwd`` with
    per-channel gates that also keeps, in the returned workspace, what
    ``chunk_bwd_kept`` needs. Returns (o [B, T, H, dv] float32,
    S_T [N, H, dk, dv] float32, workspace)."""
    if q.dim() != 4:
        raise ValueError('q must be [B, T, H, dk]')
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    code = _dtype_code(q)
    for name, t, d in (('q', q, dk), ('k', k, dk), ('v', v, dv), ('b', b, dk), ('w', w, dv)):
        _check(t, name, (B, T, H, d), dt, dev)
    _check(log_alpha, 'log_alpha', (B, T, H, dk), torch.float32, dev)
    N = _seq_count(cu_seqlens, B, dev)
    if S0 is not None:
        _check(S0, 'S0', (N, H, dk, dv), torch.float32, dev)
    o = torch.empty((B, T, H, dv), dtype=torch.float32, device=dev)
    ST = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
    need = bwd_workspace_bytes(B, T, N, H, dk, dv, dt, cu_seqlens is not None)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    set_stream()
    st = _lib.gdn2_chunk_fwd_keep(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(b), _ptr(w), _ptr(S0), _ptr(o),
                                  _ptr(ST), _ptr(cu_seqlens), B, T, N, H, dk, dv, code, GDN2_F32, _ptr(workspace),
                                  workspace.numel() * workspace.element_size())
    if st != GDN2_OK:
        raise Gdn2Error(st, 'gdn2_chunk_fwd_keep')
    return o, ST, workspace


def chunk_bwd_kept(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, log_alpha: torch.Tensor,
                   b: torch.Tensor, w: torch.Tensor, S0: Optional[torch.Tensor], dO: torch.Tensor,
                   dST: Optional[torch.Tensor] = None, cu_seqlens: Optional[torch.Tensor] = None, *,
                   workspace: torch.Tensor) -> dict:
    """``chunk_bwd`` from what the last ``chunk_fwd_keep`` on the same inputs
    left in ``workspace`` (gdn2_chunk_bwd_kept): the same gradients without
    running the forward again."""
    return _bwd('gdn2_chunk_bwd_kept', q, k, v, log_alpha, b, w, S0, dO, dST, cu_seqlens, workspace, True)
