"""fp64 CPU oracle for the input prologue of the Gated DeltaNet-2 mixer
(test infrastructure: only the tests, the smoke check and the benchmark's
CPU-baseline leg use it).

The layer's first two steps, as the guide lays them out (aifetchly-blog.pages.dev,
"Gated DeltaNet-2 Guide", the "Architectural Workflow" diagram, steps 1 and 2,
and section "2. Normalization and Short Convolutions"):

* q, k and v each pass through a short causal depthwise convolution of kernel
  size 4 (ShortConv); q and k are then scaled to unit L2 norm;
* the erase and write gates are the logistic sigmoid of their projections.

The projections themselves (W_q x, ...) are outside the mixer: this prologue
takes their outputs ("raw" q, k, v and the gate logits). The decay log-alpha
is passed through unchanged (the pages do not say how alpha is produced).

Readings where the pages leave a step open:

* The guide's code builds ShortConv as a one-dimensional convolution with one
  group per channel, padding of kernel - 1 on both sides, and keeps the first
  `seq_len` outputs ("End-to-End PyTorch Implementation", ShortConvolution).
  That is a cross-correlation over the current and three previous tokens,
  tap 3 on the current one, plus a per-channel bias (the convolution's
  default), with no activation after it.
* Unit norm as in that code's normalisation call: x / max(||x||_2, 1e-12).
* Tokens before a sequence's start are zero (the padding), unless a
  convolution history (the three raw inputs before the start, oldest first)
  is given: the state a caller carries from one call to the next, as it does
  for S0.

Everything here is plain numpy in float64, one step at a time.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from . import decode_step, forward

KERNEL = 4      # ShortConv kernel size (guide, section "2. Normalization and Short Convolutions")
HIST = KERNEL - 1
NORM_EPS = 1e-12


def _segments(tokens: int, cu_seqlens, B):
    if cu_seqlens is not None:
        cu = [int(x) for x in cu_seqlens]
        assert cu[0] == 0 and cu[-1] == tokens
        return list(zip(cu[:-1], cu[1:]))
    n = 1 if B is None else int(B)
    T = tokens // n
    assert T * n == tokens
    return [(i * T, (i + 1) * T) for i in range(n)]


def short_conv(x, weight, bias=None, cu_seqlens=None, B: Optional[int] = None, history=None):
    """Causal depthwise convolution of kernel 4 along the token axis.

    x: [tokens, H, d] (sequences packed along tokens, split by ``cu_seqlens``
    or into ``B`` equal rows); weight: [H*d, 4], tap 3 on the current token;
    bias: [H*d] or None; history: [N, H, 3, d] raw inputs before each
    sequence's start (oldest first) or None for zeros.
    Returns (y [tokens, H, d], new history [N, H, 3, d]: the last three raw
    inputs of each sequence, reaching back into the history when it is short).
    """
    x = np.asarray(x, dtype=np.float64)
    tokens, H, d = x.shape
    wt = np.asarray(weight, dtype=np.float64).reshape(H, d, KERNEL)
    bs = np.zeros((H, d)) if bias is None else np.asarray(bias, dtype=np.float64).reshape(H, d)
    segs = _segments(tokens, cu_seqlens, B)
    y = np.empty_like(x)
    hist_out = np.empty((len(segs), H, HIST, d))
    for i, (t0, t1) in enumerate(segs):
        if history is None:
            before = np.zeros((HIST, H, d))
        else:
            before = np.transpose(np.asarray(history, dtype=np.float64)[i], (1, 0, 2))   # [3, H, d]
        ext = np.concatenate([before, x[t0:t1]], axis=0)    # token t of the sequence is ext[t + 3]
        for t in range(t1 - t0):
            acc = bs.copy()
            for j in range(KERNEL):
                acc += wt[:, :, j] * ext[t + j]              # ext[t + j] is token t - 3 + j
            y[t0 + t] = acc
        hist_out[i] = np.transpose(ext[-HIST:], (1, 0, 2))
    return y, hist_out


def l2_normalize(x):
    """x / max(||x||_2, 1e-12) over the last axis."""
    x = np.asarray(x, dtype=np.float64)
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return x / np.maximum(n, NORM_EPS)


def sigmoid(x):
    """The logistic function 1 / (1 + e^-x), evaluated without overflow."""
    x = np.asarray(x, dtype=np.float64)
    e = np.exp(-np.abs(x))
    return np.where(x >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def prologue(q_raw, k_raw, v_raw, conv_w, conv_b, b_logit, w_logit, cu_seqlens=None, B=None, conv_in=None):
    """The mixer's inputs from the projections' outputs.

    conv_w / conv_b / conv_in are dicts keyed 'q', 'k', 'v' (conv_b and
    conv_in may be None, or hold None). Returns (q, k, v, b, w, conv_out)
    with conv_out a dict of new histories.
    """
    hist = {}
    out = {}
    for name, x in (('q', q_raw), ('k', k_raw), ('v', v_raw)):
        bias = None if conv_b is None else conv_b.get(name)
        h_in = None if conv_in is None else conv_in.get(name)
        out[name], hist[name] = short_conv(x, conv_w[name], bias, cu_seqlens, B, h_in)
    q = l2_normalize(out['q'])
    k = l2_normalize(out['k'])
    return q, k, out['v'], sigmoid(b_logit), sigmoid(w_logit), hist


def forward_prologue(q_raw, k_raw, v_raw, conv_w, conv_b, log_alpha, b_logit, w_logit, S0=None,
                     cu_seqlens=None, B: Optional[int] = None, conv_in=None, nthreads: int = 1,
                     want_o: bool = True):
    """Prologue, then the token recurrence. Returns (o, S_T, conv_out)."""
    q, k, v, b, w, hist = prologue(q_raw, k_raw, v_raw, conv_w, conv_b, b_logit, w_logit, cu_seqlens, B, conv_in)
    o, ST = forward(q, k, v, log_alpha, b, w, S0=S0, cu_seqlens=cu_seqlens, B=B, nthreads=nthreads, want_o=want_o)
    return o, ST, hist


def decode_step_prologue(q_raw, k_raw, v_raw, conv_w, conv_b, log_alpha, b_logit, w_logit, S, conv_state,
                         nthreads: int = 1):
    """One decode step from raw inputs [N, H, d] and the convolution history.

    conv_state: dict 'q','k','v' -> [N, H, 3, d]. Returns
    (o [N, H, dv], S_new, new conv_state).
    """
    N = np.asarray(q_raw).shape[0]
    cu = np.arange(N + 1)
    q, k, v, b, w, hist = prologue(q_raw, k_raw, v_raw, conv_w, conv_b, b_logit, w_logit,
                                   cu_seqlens=cu, conv_in=conv_state)
    o, Sn = decode_step(q, k, v, log_alpha, b, w, S, nthreads=nthreads)
    return o, Sn, hist
