"""Seeded synthetic inputs for the Gated DeltaNet-2 token mixer.

This module is shared by the tests, the benchmark and the oracle checks. It
holds none of the mixer's arithmetic: it only draws random numbers and applies
the input transforms that the pages put in front of the mixer (L2-normalised
q and k, sigmoid gates b and w, a non-positive log-decay), then rounds to the
working dtype.

Recipe (all draws are float32 from numpy's PCG64 `default_rng`):

* Every (sequence i, token block j) of 1024 tokens has its own stream
  ``default_rng([seed, i, j])``. Within a block the draws come in this order,
  each of shape ``[block_len, H, d]``: q, k, v, x_alpha, x_b, x_w, then for
  collapsed heads beta and a (shape ``[block_len, H_c]``). Any token range can
  therefore be regenerated on its own, and blocks are drawn in parallel.
* q, k ~ N(0, 1), L2-normalised over the key axis (in float64, then rounded).
* v ~ N(0, 1).
* log_alpha = -softplus(x_alpha), x_alpha ~ N(-3, 1), kept float32.
* b = sigmoid(x_b), w = sigmoid(x_w), x ~ N(0, 1).
* Collapsed heads (scalar gates): b = w = beta broadcast over channels with
  beta = sigmoid(N(0,1)); log_alpha = -softplus(N(-3,1)) broadcast over d_k.
* S0 ~ N(0, s0_std) float32 per sequence, stream ``default_rng([seed, i, 2**20])``.
* Variable lengths: ``default_rng([seed, 2**21]).integers(lo, hi, endpoint=True)``.
* Decode step s: per-step stream ``default_rng([seed, 2**22, s])`` drawing
  q, k, v, x_alpha, x_b, x_w of shape ``[N, H, d]``; the resident state is
  drawn from ``default_rng([seed, 2**22, 0])``.

bf16 rounding is round-to-nearest-even on the float32 bit pattern; the arrays
returned are float32 holding exactly the values the GPU receives.
"""
from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor
from typing import Optional

import numpy as np

BLOCK = 1024  # tokens per independent random stream


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 value (ties to even)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are already bf16-representable."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _l2n(x: np.ndarray) -> np.ndarray:
    x64 = x.astype(np.float64)
    return (x64 / np.sqrt(np.sum(x64 * x64, axis=-1, keepdims=True))).astype(np.float32)


def _softplus(x: np.ndarray) -> np.ndarray:
    return np.logaddexp(np.float32(0), x).astype(np.float32)


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return (1.0 / (1.0 + np.exp(-x.astype(np.float64)))).astype(np.float32)


@dataclasses.dataclass
class Prefill:
    """One packed prefill batch. Token tensors are ``[tokens, H, d]`` float32."""
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    log_alpha: np.ndarray
    b: np.ndarray
    w: np.ndarray
    S0: Optional[np.ndarray]      # [N, H, dk, dv] float32 or None (zeros)
    cu_seqlens: np.ndarray        # [N+1] int32 token offsets
    B: int                        # batch rows when uniform, else 1
    T: int                        # tokens per row (uniform) or total tokens
    H: int
    dk: int
    dv: int
    dtype: str                    # 'bf16' or 'f32'
    varlen: bool

    @property
    def N(self) -> int:
        return len(self.cu_seqlens) - 1

    @property
    def tokens(self) -> int:
        return int(self.cu_seqlens[-1])


def _draw_block(seed, i, j, n, H, dk, dv, dtype, collapsed):
    rng = np.random.default_rng([seed, i, j])
    f = np.float32
    q = rng.standard_normal((n, H, dk), dtype=f)
    k = rng.standard_normal((n, H, dk), dtype=f)
    v = rng.standard_normal((n, H, dv), dtype=f)
    xa = rng.standard_normal((n, H, dk), dtype=f) - f(3.0)
    xb = rng.standard_normal((n, H, dk), dtype=f)
    xw = rng.standard_normal((n, H, dv), dtype=f)
    q, k = _l2n(q), _l2n(k)
    la = -_softplus(xa)
    b, w = _sigmoid(xb), _sigmoid(xw)
    if collapsed:
        h0 = H - collapsed
        beta = _sigmoid(rng.standard_normal((n, collapsed), dtype=f))
        a = -_softplus(rng.standard_normal((n, collapsed), dtype=f) - f(3.0))
        b[:, h0:, :] = beta[:, :, None]
        w[:, h0:, :] = beta[:, :, None]
        la[:, h0:, :] = a[:, :, None]
    if dtype == 'bf16':
        q, k, v, b, w = (bf16_round(t) for t in (q, k, v, b, w))
    return q, k, v, la, b, w


def prefill(seed: int, lengths, H: int, dk: int, dv: int, dtype: str = 'bf16',
            s0_std: float = 0.0, collapsed: int = 0, uniform: bool = True,
            threads: int = 8) -> Prefill:
    """Generate a packed batch of sequences with the given lengths.

    ``uniform=True`` means the batch is B equal rows of T tokens (no cu_seqlens
    at the C-ABI); ``collapsed`` is the number of trailing heads whose gates
    are scalar per token (b = w = beta, scalar alpha).
    """
    lengths = [int(x) for x in lengths]
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    total = int(cu[-1])
    out = {name: np.empty((total, H, d), np.float32)
           for name, d in (('q', dk), ('k', dk), ('v', dv), ('la', dk), ('b', dk), ('w', dv))}
    jobs = []
    for i, L in enumerate(lengths):
        for j in range(0, (L + BLOCK - 1) // BLOCK):
            jobs.append((i, j, int(cu[i]) + j * BLOCK, min(BLOCK, L - j * BLOCK)))

    def run(job):
        i, j, t0, n = job
        arrs = _draw_block(seed, i, j, n, H, dk, dv, dtype, collapsed)
        for name, a in zip(('q', 'k', 'v', 'la', 'b', 'w'), arrs):
            out[name][t0:t0 + n] = a

    with ThreadPoolExecutor(max(1, threads)) as ex:
        list(ex.map(run, jobs))
    S0 = None
    if s0_std > 0:
        S0 = np.empty((len(lengths), H, dk, dv), np.float32)
        for i in range(len(lengths)):
            rng = np.random.default_rng([seed, i, 2 ** 20])
            S0[i] = rng.standard_normal((H, dk, dv), dtype=np.float32) * np.float32(s0_std)
    if uniform:
        assert len(set(lengths)) == 1
    return Prefill(q=out['q'], k=out['k'], v=out['v'], log_alpha=out['la'], b=out['b'],
                   w=out['w'], S0=S0, cu_seqlens=cu, B=len(lengths) if uniform else 1,
                   T=lengths[0] if uniform else total, H=H, dk=dk, dv=dv, dtype=dtype,
                   varlen=not uniform)


def varlen_lengths(seed: int, n: int, lo: int, hi: int) -> list:
    return [int(x) for x in np.random.default_rng([seed, 2 ** 21]).integers(lo, hi, size=n, endpoint=True)]


@dataclasses.dataclass
class DecodeStep:
    q: np.ndarray          # [N, H, dk]
    k: np.ndarray
    v: np.ndarray          # [N, H, dv]
    log_alpha: np.ndarray  # [N, H, dk] float32
    b: np.ndarray
    w: np.ndarray


def decode_state(seed: int, N: int, H: int, dk: int, dv: int, s0_std: float = 0.02) -> np.ndarray:
    rng = np.random.default_rng([seed, 2 ** 22, 0])
    return rng.standard_normal((N, H, dk, dv), dtype=np.float32) * np.float32(s0_std)


def decode_step(seed: int, step: int, N: int, H: int, dk: int, dv: int,
                dtype: str = 'bf16') -> DecodeStep:
    rng = np.random.default_rng([seed, 2 ** 22, step])
    f = np.float32
    q = _l2n(rng.standard_normal((N, H, dk), dtype=f))
    k = _l2n(rng.standard_normal((N, H, dk), dtype=f))
    v = rng.standard_normal((N, H, dv), dtype=f)
    la = -_softplus(rng.standard_normal((N, H, dk), dtype=f) - f(3.0))
    b = _sigmoid(rng.standard_normal((N, H, dk), dtype=f))
    w = _sigmoid(rng.standard_normal((N, H, dv), dtype=f))
    if dtype == 'bf16':
        q, k, v, b, w = (bf16_round(t) for t in (q, k, v, b, w))
    return DecodeStep(q=q, k=k, v=v, log_alpha=la, b=b, w=w)


# The five workloads, by name. Sizes follow the configuration list that the
# measurements are quoted on; `seed` doubles as the workload index.
WORKLOADS = {
    'tiny': dict(seed=0, B=1, T=128, H=1, dk=16, dv=16, dtype='f32', s0_std=0.0),
    'prefill_b4_t4096': dict(seed=1, B=4, T=4096, H=16, dk=128, dv=128, dtype='bf16', s0_std=0.0),
    'prefill_t65536': dict(seed=2, B=1, T=65536, H=16, dk=128, dv=128, dtype='bf16', s0_std=0.02),
    'decode_n256': dict(seed=3, N=256, H=16, dk=128, dv=128, dtype='bf16', steps=1000, s0_std=0.02),
    # a state (1 GiB) four times the size of the last-level cache
    'decode_n1024': dict(seed=5, N=1024, H=16, dk=128, dv=128, dtype='bf16', steps=20, s0_std=0.02),
    'varlen_32seq': dict(seed=4, n_seqs=32, lo=512, hi=16384, H=32, dk=128, dv=128,
                         dtype='bf16', s0_std=0.02, collapsed=16),
}


def workload(name: str, threads: int = 8) -> Prefill:
    """Full-size prefill workload by name (not for the decode workload)."""
    c = WORKLOADS[name]
    if name == 'varlen_32seq':
        lens = varlen_lengths(c['seed'], c['n_seqs'], c['lo'], c['hi'])
        return prefill(c['seed'], lens, c['H'], c['dk'], c['dv'], c['dtype'], c['s0_std'],
                       collapsed=c['collapsed'], uniform=False, threads=threads)
    return prefill(c['seed'], [c['T']] * c['B'], c['H'], c['dk'], c['dv'], c['dtype'],
                   c['s0_std'], uniform=True, threads=threads)


# ---- inputs for the fused prologue (ShortConv, L2 norm, sigmoid gates) ----
# Raw inputs are what the projections would hand the mixer: q, k, v before
# the short convolution and the gate logits before the sigmoid.
#
# Recipe:
# * per (sequence i, 1024-token block j) stream ``default_rng([seed, i, j, 3])``
#   drawing, each ``[block_len, H, d]``: q_raw, k_raw, v_raw ~ N(0, 1),
#   x_alpha ~ N(-3, 1) (log_alpha = -softplus(x_alpha), float32), b and w
#   logits ~ N(0, 1);
# * convolution taps ~ U(-1/2, 1/2) ``[H*d, 4]`` and biases ~ U(-1/2, 1/2)
#   ``[H*d]`` for q, k, v in that order from ``default_rng([seed, 2**23])``
#   (the default initialisation bound of a one-channel, kernel-4 convolution);
# * convolution history (three raw inputs before each sequence's start, oldest
#   first) ~ N(0, 1) ``[H, 3, d]`` per sequence, q, k, v in that order, from
#   ``default_rng([seed, i, 2**24])``;
# * bf16 workloads round the raw inputs, logits and history to bf16 (taps,
#   biases and log_alpha stay float32).
# Decode: the step-s stream ``default_rng([seed, 2**25, s])`` draws q_raw,
# k_raw, v_raw, x_alpha, b and w logits ``[N, H, d]``; the resident state
# and the history come from ``default_rng([seed, 2**25, 0])``.

CONV_K = 4


@dataclasses.dataclass
class PrologueBatch:
    q_raw: np.ndarray             # [tokens, H, dk]
    k_raw: np.ndarray
    v_raw: np.ndarray             # [tokens, H, dv]
    log_alpha: np.ndarray         # [tokens, H, dk] float32
    b_logit: np.ndarray           # [tokens, H, dk]
    w_logit: np.ndarray           # [tokens, H, dv]
    conv_w: dict                  # 'q','k','v' -> [H*d, 4] float32
    conv_b: Optional[dict]        # 'q','k','v' -> [H*d] float32, or None
    conv_in: Optional[dict]       # 'q','k','v' -> [N, H, 3, d], or None (zeros)
    S0: Optional[np.ndarray]
    cu_seqlens: np.ndarray
    B: int
    T: int
    H: int
    dk: int
    dv: int
    dtype: str
    varlen: bool

    @property
    def N(self) -> int:
        return len(self.cu_seqlens) - 1

    @property
    def tokens(self) -> int:
        return int(self.cu_seqlens[-1])


def conv_params(seed: int, H: int, dk: int, dv: int, bias: bool = True):
    rng = np.random.default_rng([seed, 2 ** 23])
    f = np.float32
    w = {n: rng.uniform(-0.5, 0.5, (H * d, CONV_K)).astype(f) for n, d in (('q', dk), ('k', dk), ('v', dv))}
    b = {n: rng.uniform(-0.5, 0.5, H * d).astype(f) for n, d in (('q', dk), ('k', dk), ('v', dv))}
    return w, (b if bias else None)


def _conv_history(seed, i, H, dk, dv, dtype):
    rng = np.random.default_rng([seed, i, 2 ** 24])
    f = np.float32
    h = {n: rng.standard_normal((H, CONV_K - 1, d), dtype=f) for n, d in (('q', dk), ('k', dk), ('v', dv))}
    if dtype == 'bf16':
        h = {n: bf16_round(a) for n, a in h.items()}
    return h


def prologue_prefill(seed: int, lengths, H: int, dk: int, dv: int, dtype: str = 'bf16',
                     s0_std: float = 0.0, uniform: bool = True, conv_bias: bool = True,
                     conv_history: bool = False, threads: int = 8) -> PrologueBatch:
    lengths = [int(x) for x in lengths]
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    total = int(cu[-1])
    names = (('q', dk), ('k', dk), ('v', dv), ('la', dk), ('xb', dk), ('xw', dv))
    out = {name: np.empty((total, H, d), np.float32) for name, d in names}
    jobs = []
    for i, L in enumerate(lengths):
        for j in range(0, (L + BLOCK - 1) // BLOCK):
            jobs.append((i, j, int(cu[i]) + j * BLOCK, min(BLOCK, L - j * BLOCK)))

    def run(job):
        i, j, t0, n = job
        rng = np.random.default_rng([seed, i, j, 3])
        f = np.float32
        arrs = {name: rng.standard_normal((n, H, d), dtype=f) for name, d in names}
        arrs['la'] = -_softplus(arrs['la'] - f(3.0))
        if dtype == 'bf16':
            for name in ('q', 'k', 'v', 'xb', 'xw'):
                arrs[name] = bf16_round(arrs[name])
        for name, a in arrs.items():
            out[name][t0:t0 + n] = a

    with ThreadPoolExecutor(max(1, threads)) as ex:
        list(ex.map(run, jobs))
    cw, cb = conv_params(seed, H, dk, dv, conv_bias)
    conv_in = None
    if conv_history:
        hs = [_conv_history(seed, i, H, dk, dv, dtype) for i in range(len(lengths))]
        conv_in = {n: np.stack([h[n] for h in hs]) for n in ('q', 'k', 'v')}
    S0 = None
    if s0_std > 0:
        S0 = np.empty((len(lengths), H, dk, dv), np.float32)
        for i in range(len(lengths)):
            rng = np.random.default_rng([seed, i, 2 ** 20])
            S0[i] = rng.standard_normal((H, dk, dv), dtype=np.float32) * np.float32(s0_std)
    if uniform:
        assert len(set(lengths)) == 1
    return PrologueBatch(q_raw=out['q'], k_raw=out['k'], v_raw=out['v'], log_alpha=out['la'],
                         b_logit=out['xb'], w_logit=out['xw'], conv_w=cw, conv_b=cb, conv_in=conv_in,
                         S0=S0, cu_seqlens=cu, B=len(lengths) if uniform else 1,
                         T=lengths[0] if uniform else total, H=H, dk=dk, dv=dv, dtype=dtype,
                         varlen=not uniform)


def prologue_decode_state(seed: int, N: int, H: int, dk: int, dv: int, dtype: str = 'bf16',
                          s0_std: float = 0.02):
    """(S [N, H, dk, dv] float32, conv history dict 'q','k','v' -> [N, H, 3, d])."""
    rng = np.random.default_rng([seed, 2 ** 25, 0])
    f = np.float32
    S = rng.standard_normal((N, H, dk, dv), dtype=f) * f(s0_std)
    h = {n: rng.standard_normal((N, H, CONV_K - 1, d), dtype=f) for n, d in (('q', dk), ('k', dk), ('v', dv))}
    if dtype == 'bf16':
        h = {n: bf16_round(a) for n, a in h.items()}
    return S, h


def prologue_decode_step(seed: int, step: int, N: int, H: int, dk: int, dv: int, dtype: str = 'bf16'):
    """(q_raw, k_raw, v_raw, log_alpha, b_logit, w_logit), each [N, H, d]."""
    rng = np.random.default_rng([seed, 2 ** 25, step])
    f = np.float32
    arrs = [rng.standard_normal((N, H, d), dtype=f) for d in (dk, dk, dv, dk, dk, dv)]
    arrs[3] = -_softplus(arrs[3] - f(3.0))
    if dtype == 'bf16':
        arrs = [a if i == 3 else bf16_round(a) for i, a in enumerate(arrs)]
    return tuple(arrs)
