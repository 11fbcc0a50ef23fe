"""Pins for the prologue oracle (oracle/prologue.py).

Each pin takes the prologue module (or a copy with a planted mistake, see
test_oracle_mutants.py) and checks it against something other than itself:
the library routines the guide's own code is built from (a grouped 1-D
convolution with padding, the normalisation call, the logistic function),
special cases whose result is known by hand (identity and shift kernels),
and the state-passing properties a causal convolution must have.

Sources (page title, section):
  FLOW  aifetchly-blog.pages.dev, "Gated DeltaNet-2 Guide", the "Architectural
        Workflow" diagram, steps 1 (ShortConv, then L2 norm of q and k) and 2
        (sigmoid gates).
  NORM  same page, "2. Normalization and Short Convolutions": causal
        depthwise convolution of kernel size 4 on q, k, v; unit-norm q and k.
  CODE  same page, "End-to-End PyTorch Implementation": the ShortConvolution
        module (grouped Conv1d, padding kernel - 1, first seq_len outputs kept)
        and the normalisation call.
"""
from __future__ import annotations

import numpy as np
import torch
import torch.nn.functional as F

import oracle

K = 4


def _rand(rng, T, H, d):
    return rng.standard_normal((T, H, d))


def _torch_conv(x, weight, bias):
    """CODE's construction: grouped Conv1d, padding 3, first T outputs kept."""
    T, H, d = x.shape
    xt = torch.from_numpy(np.ascontiguousarray(x.reshape(T, H * d).T[None]))            # [1, C, T]
    wt = torch.from_numpy(np.ascontiguousarray(weight.reshape(H * d, 1, K)))
    bt = None if bias is None else torch.from_numpy(np.ascontiguousarray(bias.reshape(H * d)))
    y = F.conv1d(xt, wt, bt, padding=K - 1, groups=H * d)[0, :, :T]
    return y.T.numpy().reshape(T, H, d)


def _close(a, b, tol, what):
    err = float(np.max(np.abs(np.asarray(a) - np.asarray(b)))) if np.size(a) else 0.0
    assert err <= tol, f'{what}: max abs diff {err:.3e} > {tol:.1e}'


def pin_conv_matches_grouped_conv1d(P):
    """NORM + CODE: ShortConv equals the library's grouped convolution."""
    rng = np.random.default_rng(11)
    for T, H, d, with_bias in ((37, 2, 5, True), (3, 1, 4, False), (1, 3, 2, True)):
        x = _rand(rng, T, H, d)
        wgt = rng.uniform(-1, 1, (H * d, K))
        bias = rng.uniform(-1, 1, H * d) if with_bias else None
        y, _ = P.short_conv(x, wgt, bias)
        _close(y, _torch_conv(x, wgt, bias), 1e-12, f'conv T={T}')


def pin_conv_special_kernels(P):
    """Identity, one- and three-token delays, and a bias-only kernel: the
    result is known by hand, and nothing before the start leaks in."""
    rng = np.random.default_rng(12)
    T, H, d = 9, 2, 3
    x = _rand(rng, T, H, d)
    for tap, delay in ((3, 0), (2, 1), (0, 3)):
        wgt = np.zeros((H * d, K))
        wgt[:, tap] = 1.0
        y, _ = P.short_conv(x, wgt)
        want = np.zeros_like(x)
        want[delay:] = x[:T - delay]
        _close(y, want, 0.0, f'kernel with tap {tap}')
    bias = rng.uniform(-1, 1, H * d)
    y, _ = P.short_conv(x, np.zeros((H * d, K)), bias)
    _close(y, np.broadcast_to(bias.reshape(1, H, d), x.shape), 0.0, 'bias only')


def pin_conv_restarts_per_sequence(P):
    """Packed sequences are convolved independently (zero before each start)."""
    rng = np.random.default_rng(13)
    H, d = 2, 4
    lens = [5, 1, 0, 9, 2]
    cu = np.concatenate([[0], np.cumsum(lens)])
    x = _rand(rng, int(cu[-1]), H, d)
    wgt = rng.uniform(-1, 1, (H * d, K))
    bias = rng.uniform(-1, 1, H * d)
    y, hist = P.short_conv(x, wgt, bias, cu_seqlens=cu)
    for i, L in enumerate(lens):
        seg = x[cu[i]:cu[i + 1]]
        if L:
            _close(y[cu[i]:cu[i + 1]], _torch_conv(seg, wgt, bias), 1e-12, f'sequence {i}')
        want = np.zeros((3, H, d))
        take = min(3, L)
        if take:
            want[3 - take:] = seg[L - take:]
        _close(hist[i], np.transpose(want, (1, 0, 2)), 0.0, f'history out of sequence {i}')
    yb, _ = P.short_conv(x[:10], wgt, bias, B=2)
    _close(yb[:5], _torch_conv(x[:5], wgt, bias), 1e-12, 'uniform rows, row 0')
    _close(yb[5:], _torch_conv(x[5:10], wgt, bias), 1e-12, 'uniform rows, row 1')


def pin_conv_history_continues(P):
    """Splitting a sequence anywhere and passing the history gives the same
    outputs as one call, also when a piece is shorter than the history."""
    rng = np.random.default_rng(14)
    H, d = 2, 3
    wgt = rng.uniform(-1, 1, (H * d, K))
    bias = rng.uniform(-1, 1, H * d)
    x = _rand(rng, 12, H, d)
    whole, hw = P.short_conv(x, wgt, bias)
    for cuts in ((1,), (2,), (7,), (1, 2, 3), (4, 5, 11)):
        pieces, h = [], None
        edges = (0,) + cuts + (12,)
        for a, b in zip(edges[:-1], edges[1:]):
            y, h = P.short_conv(x[a:b], wgt, bias, history=h)
            pieces.append(y)
        _close(np.concatenate(pieces), whole, 1e-12, f'pieces {cuts}')
        _close(h, hw, 0.0, f'history after pieces {cuts}')
    # a history given at the start acts as three earlier tokens
    pre = _rand(rng, 3, H, d)
    y, _ = P.short_conv(x, wgt, bias, history=np.transpose(pre, (1, 0, 2))[None])
    _close(y, _torch_conv(np.concatenate([pre, x]), wgt, bias)[3:], 1e-12, 'history as earlier tokens')


def pin_l2_normalize(P):
    """CODE's normalisation call; unit norm; the zero vector stays zero."""
    rng = np.random.default_rng(15)
    x = _rand(rng, 7, 3, 5)
    x[2, 1] = 0.0
    y = P.l2_normalize(x)
    _close(y, F.normalize(torch.from_numpy(x), p=2, dim=-1).numpy(), 1e-15, 'normalize')
    n = np.linalg.norm(y, axis=-1)
    n[2, 1] = 1.0
    _close(n, np.ones_like(n), 1e-14, 'unit norm')
    _close(y[2, 1], np.zeros(5), 0.0, 'zero vector')


def pin_sigmoid(P):
    """The logistic function: library values, symmetry, the midpoint, the tails."""
    x = np.concatenate([np.linspace(-40, 40, 161), [-800.0, 800.0, 0.0]])
    y = P.sigmoid(x)
    _close(y, torch.sigmoid(torch.from_numpy(x)).numpy(), 1e-15, 'sigmoid')
    _close(y + P.sigmoid(-x), np.ones_like(x), 1e-15, 'sigma(x) + sigma(-x)')
    assert y[-1] == 0.5 and y[-3] == 0.0 and y[-2] == 1.0


def pin_prologue_feeds_mixer(P):
    """FLOW steps 1-2: the mixer runs on L2Norm(ShortConv(.)) for q and k,
    ShortConv(.) for v and sigmoid gates, each built here from library calls."""
    rng = np.random.default_rng(16)
    T, H, dk, dv = 20, 2, 4, 3
    raw = {'q': _rand(rng, T, H, dk), 'k': _rand(rng, T, H, dk), 'v': _rand(rng, T, H, dv)}
    cw = {n: rng.uniform(-0.5, 0.5, (H * x.shape[-1], K)) for n, x in raw.items()}
    cb = {n: rng.uniform(-0.5, 0.5, H * x.shape[-1]) for n, x in raw.items()}
    la = -np.logaddexp(0, rng.standard_normal((T, H, dk)) - 2.0)
    xb, xw = rng.standard_normal((T, H, dk)), rng.standard_normal((T, H, dv))
    S0 = 0.1 * rng.standard_normal((1, H, dk, dv))
    o, ST, _ = P.forward_prologue(raw['q'], raw['k'], raw['v'], cw, cb, la, xb, xw, S0=S0)
    nq = F.normalize(torch.from_numpy(_torch_conv(raw['q'], cw['q'], cb['q'])), dim=-1).numpy()
    nk = F.normalize(torch.from_numpy(_torch_conv(raw['k'], cw['k'], cb['k'])), dim=-1).numpy()
    v = _torch_conv(raw['v'], cw['v'], cb['v'])
    b = torch.sigmoid(torch.from_numpy(xb)).numpy()
    w = torch.sigmoid(torch.from_numpy(xw)).numpy()
    o2, ST2 = oracle.forward(nq, nk, v, la, b, w, S0=S0)
    _close(o, o2, 1e-12, 'o')
    _close(ST, ST2, 1e-12, 'S_T')


def pin_decode_matches_prefill(P):
    """Token-by-token decode with the convolution history carried equals one
    prefill over the same tokens (outputs, state and history)."""
    rng = np.random.default_rng(17)
    T, N, H, dk, dv = 6, 2, 2, 4, 3
    raw = {'q': _rand(rng, T * N, H, dk), 'k': _rand(rng, T * N, H, dk), 'v': _rand(rng, T * N, H, dv)}
    cw = {n: rng.uniform(-0.5, 0.5, (H * x.shape[-1], K)) for n, x in raw.items()}
    cb = {n: rng.uniform(-0.5, 0.5, H * x.shape[-1]) for n, x in raw.items()}
    la = -np.logaddexp(0, rng.standard_normal((T * N, H, dk)) - 2.0)
    xb, xw = rng.standard_normal((T * N, H, dk)), rng.standard_normal((T * N, H, dv))
    h0 = {n: rng.standard_normal((N, H, 3, x.shape[-1])) for n, x in raw.items()}
    S0 = 0.1 * rng.standard_normal((N, H, dk, dv))
    o, ST, hist = P.forward_prologue(raw['q'], raw['k'], raw['v'], cw, cb, la, xb, xw, S0=S0, B=N, conv_in=h0)
    S, h = S0.copy(), {n: a.copy() for n, a in h0.items()}
    for t in range(T):
        rows = [i * T + t for i in range(N)]
        ot, S, h = P.decode_step_prologue(raw['q'][rows], raw['k'][rows], raw['v'][rows], cw, cb, la[rows],
                                          xb[rows], xw[rows], S, h)
        _close(ot, o[rows], 1e-12, f'decode o, step {t}')
    _close(S, ST, 1e-12, 'decode state')
    for n in h:
        _close(h[n], hist[n], 0.0, f'decode history {n}')


ALL = [pin_conv_matches_grouped_conv1d, pin_conv_special_kernels, pin_conv_restarts_per_sequence,
       pin_conv_history_continues, pin_l2_normalize, pin_sigmoid, pin_prologue_feeds_mixer,
       pin_decode_matches_prefill]
