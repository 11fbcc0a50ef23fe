"""fp64 CPU oracle for the Gated DeltaNet-2 token mixer (test infrastructure).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package. The product path (the HIP library and its Python
binding) never does. The arithmetic lives in ``gdn2_oracle.c``: the plain
sequential recurrence of the Gated Delta Rule-2 (snilld.dk, section "Hvad
Gated DeltaNet-2 ændrer", update equation) with readout o_t = S_t^T q_t after
the update (aifetchly-blog.pages.dev, "Gated DeltaNet-2 Guide", layer
workflow step 4). This module only marshals numpy arrays into fp64 and calls
it. ``gdn2_oracle_bwd.c`` holds the gradients: reverse-mode differentiation
of that recurrence, token by token.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, 'gdn2_oracle.c')
_SRC_BWD = os.path.join(_HERE, 'gdn2_oracle_bwd.c')
_LIB = os.path.join(_HERE, 'libgdn2_oracle.so')
_lib = None
_variants = {}


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (-O2, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + '.tmp'
        subprocess.check_call(['gcc', '-O2', '-std=c11', '-fPIC', '-shared', '-pthread',
                               '-o', tmp, _SRC, _SRC_BWD, '-lm'])
        os.replace(tmp, _LIB)
    return _LIB


def _bind(lib):
    dp = ctypes.POINTER(ctypes.c_double)
    if hasattr(lib, 'gdn2_oracle_forward'):
        lib.gdn2_oracle_forward.argtypes = [dp] * 9 + [ctypes.POINTER(ctypes.c_int64), ctypes.c_int64] + [ctypes.c_int] * 5
        lib.gdn2_oracle_forward.restype = ctypes.c_int
        lib.gdn2_oracle_decode_step.argtypes = [dp] * 8 + [ctypes.c_int] * 5
        lib.gdn2_oracle_decode_step.restype = ctypes.c_int
    if hasattr(lib, 'gdn2_oracle_backward'):
        lib.gdn2_oracle_backward.argtypes = [dp] * 16 + [ctypes.POINTER(ctypes.c_int64), ctypes.c_int64] + [ctypes.c_int] * 5
        lib.gdn2_oracle_backward.restype = ctypes.c_int
    return lib


def _load(path: Optional[str] = None):
    """The built oracle, or (for the pin-sensitivity tests) another build of it."""
    global _lib
    if path is not None:
        if path not in _variants:
            _variants[path] = _bind(ctypes.CDLL(path))
        return _variants[path]
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


def _f64(x):
    return None if x is None else np.ascontiguousarray(x, dtype=np.float64)


def _ptr(x):
    return None if x is None else x.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def forward(q, k, v, log_alpha, b, w, S0=None, cu_seqlens=None, B: Optional[int] = None,
            nthreads: int = 1, want_o: bool = True, lib: Optional[str] = None):
    """Run the recurrence over a packed batch.

    Token tensors are ``[tokens, H, d]`` (or ``[B, T, H, d]``, which is
    flattened). ``cu_seqlens`` (length N+1) gives sequence boundaries; without
    it the leading axis of a 4-D input (or ``B``) splits the tokens into equal
    sequences. Returns ``(o [tokens, H, dv] float64 or None, S_T [N, H, dk, dv])``.
    """
    q = np.asarray(q)
    if q.ndim == 4:
        B = q.shape[0] if B is None else B
        q, k, v, log_alpha, b, w = (np.asarray(t).reshape(-1, *np.asarray(t).shape[2:])
                                    for t in (q, k, v, log_alpha, b, w))
    tokens, H, dk = q.shape
    dv = np.asarray(v).shape[-1]
    if cu_seqlens is not None:
        cu = np.ascontiguousarray(cu_seqlens, dtype=np.int64)
        N, T = len(cu) - 1, 0
        assert cu[0] == 0 and cu[-1] == tokens
    else:
        cu = None
        N = 1 if B is None else int(B)
        T = tokens // N
        assert T * N == tokens
    arrs = [_f64(t) for t in (q, k, v, log_alpha, b, w)]
    S0d = _f64(S0)
    if S0d is not None:
        assert S0d.shape == (N, H, dk, dv)
    o = np.zeros((tokens, H, dv)) if want_o else None
    ST = np.zeros((N, H, dk, dv))
    rc = _load(lib).gdn2_oracle_forward(*[_ptr(a) for a in arrs], _ptr(S0d), _ptr(o), _ptr(ST),
                                 None if cu is None else cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                 T, N, H, dk, dv, int(nthreads))
    if rc != 0:
        raise ValueError('oracle rejected its arguments')
    return o, ST


def decode_step(q, k, v, log_alpha, b, w, S, nthreads: int = 1, lib: Optional[str] = None):
    """One decode step; returns ``(o [N, H, dv], S_new [N, H, dk, dv])`` in fp64."""
    arrs = [_f64(t) for t in (q, k, v, log_alpha, b, w)]
    N, H, dk = arrs[0].shape
    dv = arrs[2].shape[-1]
    Sd = np.array(S, dtype=np.float64, copy=True, order='C')
    o = np.zeros((N, H, dv))
    rc = _load(lib).gdn2_oracle_decode_step(*[_ptr(a) for a in arrs], _ptr(Sd), _ptr(o),
                                         N, H, dk, dv, int(nthreads))
    if rc != 0:
        raise ValueError('oracle rejected its arguments')
    return o, Sd


def backward(q, k, v, log_alpha, b, w, S0, dO, dST=None, cu_seqlens=None, B: Optional[int] = None,
             nthreads: int = 1, lib: Optional[str] = None):
    """Gradients of a loss with dL/do = dO and dL/dS_T = dST (None: zero).

    Inputs as in ``forward``. Returns a dict with fp64 arrays 'q', 'k', 'v',
    'log_alpha', 'b', 'w' (shapes of those inputs) and 'S0' [N, H, dk, dv].
    """
    q = np.asarray(q)
    if q.ndim == 4:
        B = q.shape[0] if B is None else B
        q, k, v, log_alpha, b, w, dO = (np.asarray(t).reshape(-1, *np.asarray(t).shape[2:])
                                        for t in (q, k, v, log_alpha, b, w, dO))
    tokens, H, dk = q.shape
    dv = np.asarray(v).shape[-1]
    if cu_seqlens is not None:
        cu = np.ascontiguousarray(cu_seqlens, dtype=np.int64)
        N, T = len(cu) - 1, 0
        assert cu[0] == 0 and cu[-1] == tokens
    else:
        cu = None
        N = 1 if B is None else int(B)
        T = tokens // N
        assert T * N == tokens
    arrs = [_f64(t) for t in (q, k, v, log_alpha, b, w)]
    S0d, dOd, dSTd = _f64(S0), _f64(dO), _f64(dST)
    assert dOd.shape == (tokens, H, dv)
    for x in (S0d, dSTd):
        if x is not None:
            assert x.shape == (N, H, dk, dv)
    g = {name: np.zeros(a.shape) for name, a in zip(('q', 'k', 'v', 'log_alpha', 'b', 'w'), arrs)}
    g['S0'] = np.zeros((N, H, dk, dv))
    rc = _load(lib).gdn2_oracle_backward(*[_ptr(a) for a in arrs], _ptr(S0d), _ptr(dOd), _ptr(dSTd),
                                         _ptr(g['q']), _ptr(g['k']), _ptr(g['v']), _ptr(g['log_alpha']),
                                         _ptr(g['b']), _ptr(g['w']), _ptr(g['S0']),
                                         None if cu is None else cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                         T, N, H, dk, dv, int(nthreads))
    if rc != 0:
        raise ValueError('oracle rejected its arguments')
    return g
