#!/usr/bin/env python3
"""Benchmark of the Gated DeltaNet-2 token mixer on one MI355X.

Headline: prefill tokens/s on the long-context workload (B=1, H=16, T=65536,
d_k=d_v=128, bf16 q/k/v/b/w, fp32 log alpha, fp32 state and output, S0 ~
N(0, 0.02)). One step = one gdn2_chunk_fwd call over the whole batch (chunk
prep + sequential state pass). The decode workload (256 sequences x 16 heads,
fp32 state resident, 1000 single-token steps with fresh inputs) is measured in
the same run and reported under "decode". Also reported: the same prefill with
scalar gates ("gate_forms": the KDA and Gated DeltaNet layouts), with chunks
of 32, 64 and 128 tokens ("chunk_sizes": latency, throughput and peak device
memory of each), on the layer's raw inputs with the short convolution, unit
norm and sigmoids fused in ("prologue_form", for prefill and decode), and the
backward of the same prefill ("backward": all input gradients from seeded dO
and dS_T).

Prints ONE JSON line. Inputs are synthetic and seeded (gdn2_inputs), resident
in HBM before timing starts. Per-kernel durations come from HIP events that
the library records on its stream during the timed region; the roofline uses
algorithmic bytes (what the method must read and write), not measured traffic.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0           # MI355X HBM3E, GB/s
METRIC = 'GDN-2 prefill tokens/s (H=16,d=128,T=64K); decode steps/s; % of roofline'


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def src_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, 'gated_delta_rule_wy_amd', 'csrc')
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), 'rb') as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def traffic_for(kernel: str, workload: str):
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, 'profiles', 'traffic.json')
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    e = d.get(f'{kernel}@{workload}')
    if not e or e.get('source_sha') != src_hash():
        return None
    return e['fetch_bytes'] + e['write_bytes']


def step_traffic(workload):
    """Counter HBM bytes of the prefill step (preparation + pass), or None."""
    t = [traffic_for(k, workload) for k in ('gdn2_chunk_prep', 'gdn2_chunk_pass')]
    return None if None in t else sum(t)


def mfma_summary(model_flop_frac, ms_per_step):
    """Matrix-core use of the T = 64K prefill step: the algorithmic (model)
    FLOP fraction measured here, and from the committed counter summary
    (when it was taken on the current kernel sources, else null) the
    rocprof MFMA-busy fraction of each kernel and the issued MFMA FLOPs per
    step over this step's time."""
    out = {'peak_tflops': PEAK_MFMA_F16_TFLOPS, 'model_flop_frac': model_flop_frac, 'busy_frac': None,
           'issued_flop_frac': None}
    path = os.path.join(ROOT, 'profiles', 'mfma.json')
    if os.path.exists(path):
        with open(path) as f:
            d = json.load(f)
        if d.get('source_sha') == src_hash():
            out['busy_frac'] = d.get('busy_frac')
            fl = d.get('issued_flop_per_step')
            if fl:
                out['issued_flop_frac'] = round(fl / (ms_per_step * 1e-3) / 1e12 / PEAK_MFMA_F16_TFLOPS, 4)
            out['normalisation'] = d.get('normalisation')
    return out


def roofline(kernel, alg_bytes, avg_ms, workload):
    achieved = alg_bytes / (avg_ms * 1e-3) / 1e9
    return {'bound': 'hbm', 'kernel': kernel, 'achieved': round(achieved, 1), 'peak': PEAK_HBM_GBS,
            'unit': 'GB/s', 'frac': round(achieved / PEAK_HBM_GBS, 4),
            'traffic': traffic_for(kernel, workload), 'alg_bytes_per_launch': int(alg_bytes),
            'avg_launch_ms': round(avg_ms, 5)}


def nthreads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def bench_prefill(args, torch, gdn2, gi):
    name = 'prefill_t65536'
    c = gi.WORKLOADS[name]
    B, T, H, dk, dv = c['B'], c['T'], c['H'], c['dk'], c['dv']
    t0 = time.time()
    p = gi.workload(name, threads=nthreads())
    log(f'[bench] generated {name} in {time.time() - t0:.1f}s')
    dev = torch.device('cuda:0')
    to = lambda x, dt: torch.from_numpy(x).to(dev).to(dt).reshape(B, T, H, x.shape[-1])
    bf = torch.bfloat16
    q, k, v, b, w = (to(x, bf) for x in (p.q, p.k, p.v, p.b, p.w))
    la = to(p.log_alpha, torch.float32)
    S0 = torch.from_numpy(p.S0).to(dev)
    o = torch.empty(B, T, H, dv, device=dev)
    ST = torch.empty(B, H, dk, dv, device=dev)
    ws = torch.empty(gdn2.workspace_bytes(B, T, B, H, dk, dv, bf, False), dtype=torch.uint8, device=dev)
    run = lambda: gdn2.chunk_fwd(q, k, v, la, b, w, S0, out=o, final_state=ST, workspace=ws)
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    gdn2.profile_begin(args.steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        run()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    prof = gdn2.profile_end()
    ms = (t1 - t0) * 1e3 / args.steps
    log(f'[bench] prefill {ms:.3f} ms/step; kernels: ' +
        ', '.join(f'{k} {v[1] / max(1, v[0]):.4f} ms' for k, v in prof.items()))

    TH = B * T * H
    in_b = 2 if p.dtype == 'bf16' else 4
    alg = {
        # what each kernel must read or write at the least: prep reads q, k, b and
        # log alpha; the pass reads v, w and S0, writes o and S_T
        'gdn2_chunk_prep': TH * (3 * dk * in_b + dk * 4),
        'gdn2_chunk_pass': TH * (2 * dv * in_b + dv * 4) + 2 * B * H * dk * dv * 4,
    }
    avg = {k: v[1] / v[0] for k, v in prof.items() if v[0]}
    dom = max(avg, key=avg.get)
    step_bytes = sum(alg.values())
    res = {
        'ms_per_step': round(ms, 4), 'value': B * T / (ms * 1e-3),
        'roofline': roofline(dom, alg[dom], avg[dom], name),
        'step_roofline': {'bound': 'hbm', 'alg_bytes_per_step': int(step_bytes),
                          'achieved': round(step_bytes / (ms * 1e-3) / 1e9, 1), 'peak': PEAK_HBM_GBS,
                          'unit': 'GB/s', 'frac': round(step_bytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                          'traffic': step_traffic(name),
                          'traffic_ratio': (round(step_traffic(name) / step_bytes, 3)
                                            if step_traffic(name) else None)},
        'kernels_ms': {k: round(v, 5) for k, v in avg.items()},
        'model_flop_frac': round(TH * flops_per_token_head(dk, dv) / (ms * 1e-3) / 1e12 / PEAK_MFMA_F16_TFLOPS, 4),
    }

    # The same workload with gates of one value per token-head: the Kimi Delta
    # Attention form (erase and write gate = one beta) and the Gated DeltaNet
    # form (also one decay), the cases Gated DeltaNet-2 reduces to. The gate
    # values are the per-channel gates' first channel; only the timing is used.
    forms = {}
    b1 = b[..., 0].contiguous()
    la1 = la[..., 0].contiguous()
    o1 = torch.empty_like(o)       # keeps o for the parity sample below
    ST1 = torch.empty_like(ST)
    for fname, (fb, fw, fla) in (() if args.no_gate_forms else (('kda', (b1, b1, la)), ('gdn', (b1, b1, la1)))):
        frun = lambda: gdn2.chunk_fwd(q, k, v, fla, fb, fw, S0, out=o1, final_state=ST1, workspace=ws)
        for _ in range(args.warmup):
            frun()
        torch.cuda.synchronize()
        gdn2.profile_begin(args.steps)
        t0 = time.perf_counter()
        for _ in range(args.steps):
            frun()
        torch.cuda.synchronize()
        fms = (time.perf_counter() - t0) * 1e3 / args.steps
        fprof = gdn2.profile_end()
        la_b = dk * 4 if fla is la else 4
        fbytes = TH * (2 * dk * in_b + in_b + la_b) + TH * (dv * in_b + in_b + dv * 4) + 2 * B * H * dk * dv * 4
        forms[fname] = {'ms_per_step': round(fms, 4), 'value': B * T / (fms * 1e-3), 'unit': 'tokens/s',
                        'alg_bytes_per_step': int(fbytes),
                        'step_roofline_frac': round(fbytes / (fms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                        'kernels_ms': {kk: round(vv[1] / vv[0], 5) for kk, vv in fprof.items() if vv[0]}}
        log(f'[bench] prefill, {fname} gates: {fms:.3f} ms/step')
    res['gate_forms'] = forms

    # Chunk sizes (the C = 32 / 64 / 128 trade-off): latency, throughput and
    # peak device memory of the same workload, measured back to back.
    sizes = {}
    for C in (() if args.no_chunk_sizes else (64, 32, 128)):
        need = gdn2.workspace_bytes(B, T, B, H, dk, dv, bf, False, chunk=C)
        wsc = torch.empty(need, dtype=torch.uint8, device=dev)
        crun = lambda: gdn2.chunk_fwd(q, k, v, la, b, w, S0, out=o1, final_state=ST1, workspace=wsc, chunk=C)
        for _ in range(args.warmup):
            crun()
        torch.cuda.synchronize()
        gdn2.profile_begin(args.steps)
        t0 = time.perf_counter()
        for _ in range(args.steps):
            crun()
        torch.cuda.synchronize()
        cms = (time.perf_counter() - t0) * 1e3 / args.steps
        cprof = gdn2.profile_end()
        resident = sum(x.numel() * x.element_size() for x in (q, k, v, b, w, la, S0, o1, ST1))
        sizes[str(C)] = {'ms_per_step': round(cms, 4), 'value': B * T / (cms * 1e-3), 'unit': 'tokens/s',
                         'step_roofline_frac': round(step_bytes / (cms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                         'workspace_bytes': int(need), 'peak_device_bytes': int(resident + need),
                         'kernels_ms': {kk: round(vv[1] / vv[0], 5) for kk, vv in cprof.items() if vv[0]}}
        log(f'[bench] prefill, chunk {C}: {cms:.3f} ms/step; kernels: ' +
            ', '.join(f'{kk} {vv[1] / max(1, vv[0]):.4f} ms' for kk, vv in cprof.items()) +
            f'; workspace {need / 2**20:.0f} MiB')
        del wsc
    res['chunk_sizes'] = sizes
    if not args.no_prologue:
        res['prologue_form'] = bench_prefill_prologue(args, torch, gdn2, gi, ws)
    if not args.no_backward:
        res['backward'] = bench_backward(args, torch, gdn2, q, k, v, la, b, w, S0, p)

    if not args.no_cpu_baseline:
        import oracle
        n_s = args.cpu_sample_tokens
        sl = slice(0, n_s)
        nt = nthreads()
        t0 = time.perf_counter()
        o_ref, _ = oracle.forward(p.q[sl], p.k[sl], p.v[sl], p.log_alpha[sl], p.b[sl], p.w[sl], p.S0,
                                  nthreads=nt)
        dt = time.perf_counter() - t0
        res['cpu_baseline'] = {'value': round(n_s / dt, 1), 'unit': 'tokens/s', 'cores': min(nt, H),
                               'kind': 'oracle',
                               'sample': f'first {n_s} of {T} tokens, all {H} heads (one thread per head '
                                         f'chain, {min(nt, H)} chains at once), fp64; {dt:.1f}s'}
        o_gpu = o[0, :n_s].float().cpu().numpy()
        rms = float(np.sqrt(np.mean(o_ref ** 2)))
        res['parity_sample'] = {'max_abs_err_over_rms': float(np.max(np.abs(o_gpu - o_ref)) / rms),
                                'tokens': n_s}
        log(f'[bench] oracle {n_s} tokens in {dt:.1f}s; parity {res["parity_sample"]}')
    del q, k, v, b, w, la, o, ws, b1, la1, o1, ST1
    torch.cuda.empty_cache()
    return res


PEAK_MFMA_F16_TFLOPS = 2500.0   # MI355X dense f16 / bf16 matrix peak, TFLOP/s


def flops_per_token_head(dk, dv, C=64):
    """Algorithmic work of the chunk method per token and head: the state
    products (6 dk dv), the C x C blocks over dk and dv, triangular halves
    counted once (C (3 dk + 2 dv) + C^2 / 3)."""
    return 6 * dk * dv + C * (3 * dk + 2 * dv) + C * C // 3


def bench_prefill_config(args, torch, gdn2, gi, name):
    """tokens/s of one more prefill workload (its own launch configuration)."""
    c = gi.WORKLOADS[name]
    t0 = time.time()
    p = gi.workload(name, threads=nthreads())
    log(f'[bench] generated {name} ({p.tokens} tokens x {p.H} heads) in {time.time() - t0:.1f}s')
    dev = torch.device('cuda:0')
    bf = torch.bfloat16
    shp = (p.B, -1, p.H)
    to = lambda x, dt: torch.from_numpy(x).to(dev).to(dt).reshape(*shp, x.shape[-1])
    q, k, v, b, w = (to(x, bf) for x in (p.q, p.k, p.v, p.b, p.w))
    la = to(p.log_alpha, torch.float32)
    del p.q, p.k, p.v, p.b, p.w, p.log_alpha
    S0 = torch.from_numpy(p.S0).to(dev) if p.S0 is not None else None
    cu = torch.from_numpy(p.cu_seqlens).to(dev) if p.varlen else None
    o = torch.empty(*q.shape[:3], p.dv, device=dev)
    ST = torch.empty(p.N, p.H, p.dk, p.dv, device=dev)
    ws = torch.empty(gdn2.workspace_bytes(p.B, p.T, p.N, p.H, p.dk, p.dv, bf, p.varlen), dtype=torch.uint8,
                     device=dev)
    run = lambda: gdn2.chunk_fwd(q, k, v, la, b, w, S0, cu, out=o, final_state=ST, workspace=ws)
    steps = max(5, args.steps // 2) if p.varlen else args.steps
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    gdn2.profile_begin(steps)
    t0 = time.perf_counter()
    for _ in range(steps):
        run()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    prof = gdn2.profile_end()
    TH = p.tokens * p.H
    nbytes = TH * (3 * p.dk * 2 + p.dk * 4 + 2 * p.dv * 2 + p.dv * 4) + (2 if S0 is not None else 1) * \
        p.N * p.H * p.dk * p.dv * 4
    fl = TH * flops_per_token_head(p.dk, p.dv)
    log(f'[bench] {name}: {ms:.3f} ms/step, {p.tokens / (ms * 1e-3) / 1e6:.1f} M tokens/s')
    res = {'workload': name, 'tokens': p.tokens, 'H': p.H, 'sequences': p.N, 'steps': steps,
           'ms_per_step': round(ms, 4), 'value': round(p.tokens / (ms * 1e-3), 1), 'unit': 'tokens/s',
           'alg_bytes_per_step': int(nbytes),
           'step_roofline_frac': round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
           'model_flop_frac': round(fl / (ms * 1e-3) / 1e12 / PEAK_MFMA_F16_TFLOPS, 4),
           'kernels_ms': {kk: round(vv[1] / vv[0], 5) for kk, vv in prof.items() if vv[0]}}
    del q, k, v, b, w, la, o, ws, ST, S0
    torch.cuda.empty_cache()
    return res


def bench_backward(args, torch, gdn2, q, k, v, la, b, w, S0, p):
    """Gradients of a loss through the same prefill (gdn2_chunk_bwd: the
    forward again keeping chunk states, the reverse state-gradient pass and
    the per-chunk gradients), with seeded dO and dS_T."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    rng = np.random.default_rng(12345)
    dO = torch.from_numpy(rng.standard_normal((B, T, H, dv), dtype=np.float32)).to(q.device)
    dST = torch.from_numpy(rng.standard_normal((B, H, dk, dv), dtype=np.float32)).to(q.device)
    need = gdn2.lib().gdn2_chunk_bwd_workspace_bytes(B, T, B, H, dk, dv, gdn2.GDN2_BF16, 0)
    wsb = torch.empty(need, dtype=torch.uint8, device=q.device)
    run = lambda: gdn2.chunk_bwd(q, k, v, la, b, w, S0, dO, dST, workspace=wsb)
    for _ in range(args.warmup):
        g = run()
    torch.cuda.synchronize()
    gdn2.profile_begin(args.steps)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        g = run()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    prof = gdn2.profile_end()
    avg = {kk: vv[1] / vv[0] for kk, vv in prof.items() if vv[0]}
    TH = B * T * H
    # reads q, k, v, b, w (bf16), log alpha and dO (fp32); writes dq, dk, db,
    # dlog alpha, dv, dw (fp32); S0, dS_T in, dS0 out
    nbytes = TH * (3 * dk * 2 + 2 * dv * 2 + dk * 4 + dv * 4) + TH * (4 * dk * 4 + 2 * dv * 4) + 3 * B * H * dk * dv * 4
    log(f'[bench] backward {ms:.3f} ms/step; kernels: ' + ', '.join(f'{kk} {vv:.4f} ms' for kk, vv in avg.items()))
    res = {'ms_per_step': round(ms, 4), 'value': B * T / (ms * 1e-3), 'unit': 'tokens/s',
           'inputs': 'same prefill; seeded dO and dS_T; fp32 gradients',
           'alg_bytes_per_step': int(nbytes),
           'step_roofline_frac': round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
           'kernels_ms': {kk: round(vv, 5) for kk, vv in avg.items()},
           # the per-chunk gradient kernel reads and writes every per-token tensor
           'roofline': roofline('gdn2_chunk_grad', nbytes, avg['gdn2_chunk_grad'], 'backward_t65536')}
    # The training step: the forward that keeps what the backward needs
    # (gdn2_chunk_fwd_keep: o and S_T as gdn2_chunk_fwd, plus the operand
    # blocks, chunk states and corrected writes) and the backward from them
    # (gdn2_chunk_bwd_kept), against gdn2_chunk_fwd followed by gdn2_chunk_bwd.
    def train():
        gdn2.chunk_fwd_keep(q, k, v, la, b, w, S0, workspace=wsb)
        return gdn2.chunk_bwd_kept(q, k, v, la, b, w, S0, dO, dST, workspace=wsb)
    for _ in range(args.warmup):
        g = train()
    torch.cuda.synchronize()
    gdn2.profile_begin(2 * args.steps)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        g = train()
    torch.cuda.synchronize()
    tms = (time.perf_counter() - t0) * 1e3 / args.steps
    tprof = gdn2.profile_end()
    tavg = {kk: vv[1] / vv[0] for kk, vv in tprof.items() if vv[0]}
    log(f'[bench] training step (keep + kept) {tms:.3f} ms/step; kernels: ' +
        ', '.join(f'{kk} {vv:.4f} ms' for kk, vv in tavg.items()))
    fwd_bytes = TH * (3 * dk * 2 + dk * 4) + TH * (2 * dv * 2 + dv * 4) + 2 * B * H * dk * dv * 4
    res['training_step'] = {
        'ms_per_step': round(tms, 4), 'value': B * T / (tms * 1e-3), 'unit': 'tokens/s',
        'what': 'gdn2_chunk_fwd_keep then gdn2_chunk_bwd_kept (o, S_T and every gradient)',
        'alg_bytes_per_step': int(fwd_bytes + nbytes),
        'step_roofline_frac': round((fwd_bytes + nbytes) / (tms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        'kernels_ms': {kk: round(vv, 5) for kk, vv in tavg.items()}}
    if not args.no_cpu_baseline:
        import oracle
        n_s = min(T, args.cpu_sample_tokens // 4)
        sl = slice(0, n_s)
        h = lambda x: x[0, sl].float().cpu().numpy()
        t0 = time.perf_counter()
        oracle.backward(h(q), h(k), h(v), h(la), h(b), h(w), p.S0, h(dO), dST.cpu().numpy(),
                        nthreads=nthreads())
        dt = time.perf_counter() - t0
        res['cpu_baseline'] = {'value': round(n_s / dt, 1), 'unit': 'tokens/s', 'cores': min(nthreads(), H),
                               'kind': 'oracle',
                               'sample': f'first {n_s} of {T} tokens, all {H} heads, fp64 reverse sweep; {dt:.1f}s'}
    del dO, dST, wsb, g
    torch.cuda.empty_cache()
    return res


def bench_prefill_prologue(args, torch, gdn2, gi, ws):
    """The same workload in the layer's raw form: q, k, v before the short
    convolution and b, w as logits (gdn2_chunk_fwd_prologue: the convolution,
    unit norm and sigmoid run inside the mixer's kernels), with a
    convolution history in and out per sequence."""
    c = gi.WORKLOADS['prefill_t65536']
    B, T, H, dk, dv = c['B'], c['T'], c['H'], c['dk'], c['dv']
    t0 = time.time()
    p = gi.prologue_prefill(c['seed'], [T] * B, H, dk, dv, c['dtype'], c['s0_std'], conv_history=True,
                            threads=nthreads())
    dev = torch.device('cuda:0')
    bf = torch.bfloat16
    t = lambda x, d: torch.from_numpy(x).to(dev).to(d).reshape(B, T, H, x.shape[-1])
    qr, kr, vr, xb, xw = (t(x, bf) for x in (p.q_raw, p.k_raw, p.v_raw, p.b_logit, p.w_logit))
    la = t(p.log_alpha, torch.float32)
    trip = lambda d, dt: tuple(torch.from_numpy(d[n]).to(dev).to(dt) for n in ('q', 'k', 'v'))
    cw, cb, hin = trip(p.conv_w, torch.float32), trip(p.conv_b, torch.float32), trip(p.conv_in, bf)
    hout = tuple(torch.empty_like(x) for x in hin)
    S0 = torch.from_numpy(p.S0).to(dev)
    o = torch.empty(B, T, H, dv, device=dev)
    ST = torch.empty_like(S0)
    log(f'[bench] generated the raw-form workload in {time.time() - t0:.1f}s')
    run = lambda: gdn2.chunk_fwd_prologue(qr, kr, vr, la, xb, xw, cw, cb, S0, conv_state=hin, conv_state_out=hout,
                                          out=o, final_state=ST, workspace=ws)
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    gdn2.profile_begin(args.steps)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        run()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    prof = gdn2.profile_end()
    TH = B * T * H
    conv_bytes = H * (2 * dk + dv) * 5 * 4 + 2 * B * H * 3 * (2 * dk + dv) * 2   # taps, biases, history in + out
    nbytes = TH * (3 * dk * 2 + dk * 4) + TH * (2 * dv * 2 + dv * 4) + 2 * B * H * dk * dv * 4 + conv_bytes
    log(f'[bench] prefill, fused prologue: {ms:.3f} ms/step')
    del qr, kr, vr, xb, xw, la, o
    return {'ms_per_step': round(ms, 4), 'value': B * T / (ms * 1e-3), 'unit': 'tokens/s',
            'inputs': 'raw bf16 q,k,v and b,w logits; ShortConv k=4 with bias and history, L2 norm, sigmoid fused',
            'alg_bytes_per_step': int(nbytes),
            'step_roofline_frac': round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            'kernels_ms': {k: round(v[1] / v[0], 5) for k, v in prof.items() if v[0]}}


def bench_decode(args, torch, gdn2, gi, name='decode_n256', cycles=1):
    """Decode steps on the resident state. `cycles` > 1 replays the workload's
    step inputs that many times (the large state's inputs are drawn for a few
    steps only; the state, not the inputs, is what each step streams)."""
    c = gi.WORKLOADS[name]
    N, H, d = c['N'], c['H'], c['dk']
    extras = name == 'decode_n256'
    steps = args.decode_steps if extras else c['steps']
    dev = torch.device('cuda:0')
    bf = torch.bfloat16
    from concurrent.futures import ThreadPoolExecutor
    t0 = time.time()
    with ThreadPoolExecutor(nthreads()) as ex:
        host = list(ex.map(lambda s: gi.decode_step(c['seed'], s, N, H, d, d), range(1, steps + 1)))
    stack = lambda f, dt: torch.from_numpy(np.stack([getattr(h, f) for h in host])).to(dev).to(dt)
    q, k, v, b, w = (stack(f, bf) for f in ('q', 'k', 'v', 'b', 'w'))
    la = stack('log_alpha', torch.float32)
    S_np = gi.decode_state(c['seed'], N, H, d, d, c['s0_std'])
    S = torch.from_numpy(S_np).to(dev)
    o = torch.empty(N, H, d, device=dev)
    log(f'[bench] generated {steps} decode steps in {time.time() - t0:.1f}s')
    step = lambda s: gdn2.decode_step(q[s % steps], k[s % steps], v[s % steps], la[s % steps], b[s % steps],
                                      w[s % steps], S, out=o)
    timed = steps * cycles
    for s in range(min(10, steps)):
        step(s)
    torch.cuda.synchronize()
    gdn2.profile_begin(timed)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(timed):
        step(s)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    prof = gdn2.profile_end()
    n, tot = prof['gdn2_decode']
    avg = tot / n
    per_chain = 2 * d * d * 4 + (3 * d + 2 * d) * 2 + d * 4 + d * 4   # S r+w, q k b v w, log alpha, o
    res = {'metric': 'decode steps/s', 'value': timed / (t1 - t0), 'unit': 'steps/s',
           'steps': timed, 'ms_per_step': round((t1 - t0) * 1e3 / timed, 5),
           'config': {'workload': name, 'N': N, 'H': H, 'dk': d, 'dv': d,
                      'state': f'fp32 [N,H,dk,dv] resident ({N * H * d * d * 4 / 2**30:.2f} GiB), updated in place',
                      'inputs': 'bf16, fresh per step' if cycles == 1 else
                                f'bf16, {steps} distinct steps replayed {cycles} times'},
           'roofline': roofline('gdn2_decode', per_chain * N * H, avg, name)}
    log(f'[bench] decode {name}: {res["ms_per_step"]} ms/step, kernel {avg * 1e3:.1f} us')
    if not extras:
        return res
    if not args.no_prologue:
        # raw inputs (q, k, v before the short convolution, gate logits) with
        # the convolution history updated in place
        np_ = min(steps, 200)
        raw = [gi.prologue_decode_step(c['seed'], s, N, H, d, d) for s in range(1, np_ + 1)]
        rs = lambda j, dt: torch.from_numpy(np.stack([r[j] for r in raw])).to(dev).to(dt)
        qr, kr, vr, xb, xw = (rs(j, bf) for j in (0, 1, 2, 4, 5))
        lr = rs(3, torch.float32)
        _, h_np = gi.prologue_decode_state(c['seed'], N, H, d, d)
        hist = tuple(torch.from_numpy(h_np[n]).to(dev).to(bf) for n in ('q', 'k', 'v'))
        cw_np, cb_np = gi.conv_params(c['seed'], H, d, d)
        cw = tuple(torch.from_numpy(cw_np[n]).to(dev) for n in ('q', 'k', 'v'))
        cb = tuple(torch.from_numpy(cb_np[n]).to(dev) for n in ('q', 'k', 'v'))
        pstep = lambda s: gdn2.decode_step_prologue(qr[s], kr[s], vr[s], lr[s], xb[s], xw[s], S, cw, cb, hist, out=o)
        for s in range(min(10, np_)):
            pstep(s)
        torch.cuda.synchronize()
        gdn2.profile_begin(np_)
        t0 = time.perf_counter()
        for s in range(np_):
            pstep(s)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        n, tot = gdn2.profile_end()['gdn2_decode']
        pavg = tot / n
        per_pro = per_chain + 2 * 3 * 3 * d * 2   # + history of q, k, v read and written
        res['prologue_form'] = {'steps': np_, 'ms_per_step': round((t1 - t0) * 1e3 / np_, 5),
                                'value': np_ / (t1 - t0), 'unit': 'steps/s',
                                'roofline': roofline('gdn2_decode', per_pro * N * H, pavg, name + '_prologue')}
        log(f'[bench] decode, fused prologue: kernel {pavg * 1e3:.1f} us')
    if not args.no_cpu_baseline:
        import oracle
        ns = args.cpu_decode_steps
        nt = nthreads()
        S_c = S_np
        t0 = time.perf_counter()
        for s in range(ns):
            h = host[s]
            _, S_c = oracle.decode_step(h.q, h.k, h.v, h.log_alpha, h.b, h.w, S_c, nthreads=nt)
        dt = time.perf_counter() - t0
        res['cpu_baseline'] = {'value': round(ns / dt, 3), 'unit': 'steps/s', 'cores': nt, 'kind': 'oracle',
                               'sample': f'{ns} of {steps} steps over all {N * H} chains, fp64; {dt:.1f}s'}
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument('--gpus', type=int, default=1)
    ap.add_argument('--steps', type=int, default=20)
    ap.add_argument('--warmup', type=int, default=20)
    ap.add_argument('--decode-steps', type=int, default=1000)
    ap.add_argument('--cpu-sample-tokens', type=int, default=65536)
    ap.add_argument('--cpu-decode-steps', type=int, default=100)
    ap.add_argument('--no-cpu-baseline', action='store_true')
    ap.add_argument('--no-decode', action='store_true')
    ap.add_argument('--no-backward', action='store_true',
                    help='skip the backward (gradient) timing')
    ap.add_argument('--no-prologue', action='store_true',
                    help='skip the fused-prologue (raw-input) timings')
    ap.add_argument('--no-gate-forms', action='store_true',
                    help='skip the scalar-gate (KDA, Gated DeltaNet) prefill timings')
    ap.add_argument('--no-other-configs', action='store_true',
                    help='skip the B=4 x T=4096 and packed varlen (H=32) prefill timings')
    ap.add_argument('--no-chunk-sizes', action='store_true',
                    help='skip the chunk-size (32 / 64 / 128 tokens) prefill timings')
    ap.add_argument('--copy-calibration-mib', type=int, default=0,
                    help='only run a plain device copy of this many MiB (x3), to calibrate '
                         'the FETCH_SIZE / WRITE_SIZE counters; prints nothing else')
    args = ap.parse_args()
    if args.gpus != 1:
        print(f'bench.py measures one GPU only: the mixer is benchmarked on one MI355X '
              f'(--gpus {args.gpus} is not supported)', file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        src = torch.ones(n // 4, device='cuda:0')
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f'[bench] copied {args.copy_calibration_mib} MiB x3')
        return

    import gated_delta_rule_wy_amd as gdn2
    import gdn2_inputs as gi

    pre = bench_prefill(args, torch, gdn2, gi)
    out = {
        'metric': METRIC, 'value': round(pre['value'], 1), 'unit': 'tokens/s', 'n_gpus': 1,
        'steps': args.steps, 'warmup': args.warmup, 'ms_per_step': pre['ms_per_step'],
        'higher_is_better': True, 'scaling': 'weak', 'vs_baseline': None, 'dtype': 'f16',
        'data': 'synthetic',
        'config': {'workload': 'prefill_t65536', 'B': 1, 'T': 65536, 'H': 16, 'dk': 128, 'dv': 128,
                   'chunk': 64, 'inputs': 'bf16 q,k,v,b,w; fp32 log_alpha; fp32 S0, S_T and o',
                   'compute': 'f16 MFMA operands, fp32 accumulation and state'},
        'roofline': pre['roofline'],
    }
    if 'cpu_baseline' in pre:
        out['cpu_baseline'] = pre['cpu_baseline']
    out['step_roofline'] = pre['step_roofline']
    out['mfma'] = mfma_summary(pre['model_flop_frac'], pre['ms_per_step'])
    out['kernels_ms'] = pre['kernels_ms']
    out['gate_forms'] = pre['gate_forms']
    out['chunk_sizes'] = pre['chunk_sizes']
    if 'prologue_form' in pre:
        out['prologue_form'] = pre['prologue_form']
    if 'backward' in pre:
        out['backward'] = pre['backward']
    if 'parity_sample' in pre:
        out['parity_sample'] = pre['parity_sample']
    if not args.no_other_configs:
        out['other_prefill'] = [bench_prefill_config(args, torch, gdn2, gi, n)
                                for n in ('prefill_b4_t4096', 'varlen_32seq')]
    if not args.no_decode:
        out['decode'] = bench_decode(args, torch, gdn2, gi)
        out['decode_large_state'] = bench_decode(args, torch, gdn2, gi, 'decode_n1024', cycles=10)
    print(json.dumps(out), flush=True)


if __name__ == '__main__':
    main()
