"""Helpers for the GPU parity tests: move seeded inputs to the device, run the
library through its binding, and measure errors against the oracle."""
from __future__ import annotations

import os

import numpy as np
import torch

import gdn2_inputs as gi

DEV = torch.device('cuda:0')
TOL_F32 = 1e-4       # max-abs error bar for fp32 inputs
TOL_BF16 = 2e-2      # max-abs error bar, relative to the reference RMS, for bf16 inputs


def threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def dev(x, dtype):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV).to(dtype)


def tdtype(name):
    return torch.bfloat16 if name == 'bf16' else torch.float32


def run_prefill(p: gi.Prefill, S0=True, **kw):
    import gated_delta_rule_wy_amd as gdn2
    dt = tdtype(p.dtype)
    shp = (p.B, -1, p.H)
    t = lambda x, d: dev(x, d).reshape(*shp, x.shape[-1])
    q, k, v, b, w = (t(x, dt) for x in (p.q, p.k, p.v, p.b, p.w))
    la = t(p.log_alpha, torch.float32)
    s0 = dev(p.S0, torch.float32) if (S0 and p.S0 is not None) else None
    cu = dev(p.cu_seqlens, torch.int32) if p.varlen else None
    o, ST = gdn2.chunk_fwd(q, k, v, la, b, w, s0, cu, **kw)
    torch.cuda.synchronize()
    return o.reshape(-1, p.H, p.dv).cpu().numpy(), None if ST is None else ST.cpu().numpy()


def oracle_prefill(p: gi.Prefill, seqs=None):
    import oracle
    if seqs is None:
        return oracle.forward(p.q, p.k, p.v, p.log_alpha, p.b, p.w, p.S0,
                              cu_seqlens=p.cu_seqlens, nthreads=threads())
    # a subset of sequences, each run on its own (sequences are independent)
    outs = {}
    for i in seqs:
        s = slice(int(p.cu_seqlens[i]), int(p.cu_seqlens[i + 1]))
        S0 = None if p.S0 is None else p.S0[i:i + 1]
        outs[i] = oracle.forward(p.q[s], p.k[s], p.v[s], p.log_alpha[s], p.b[s], p.w[s], S0,
                                 nthreads=threads())
    return outs


def rel_max(x, ref):
    rms = float(np.sqrt(np.mean(np.square(ref)))) if np.size(ref) else 0.0
    err = float(np.max(np.abs(x - ref))) if np.size(ref) else 0.0
    return err / rms if rms > 0 else err, err, rms


def assert_close(x, ref, dtype, what, quiet=False):
    """fp32 inputs: max-abs <= 1e-4. bf16 inputs: max-abs <= 2e-2 * RMS(ref)."""
    assert np.all(np.isfinite(x)), f'{what}: non-finite values'
    r, err, rms = rel_max(x, ref)
    if dtype == 'f32':
        assert err <= TOL_F32, f'{what}: max abs error {err:.3e} > {TOL_F32}'
    else:
        assert r <= TOL_BF16, f'{what}: max abs error {err:.3e} = {r:.3e} x RMS {rms:.3e} > {TOL_BF16}'
    if not quiet:
        print(f'{what}: max abs err {err:.3e}, / RMS {r:.3e}', flush=True)
    return r
