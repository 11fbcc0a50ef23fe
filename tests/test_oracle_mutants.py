"""Pin sensitivity: plant plausible mistakes in copies of the oracle's C source
(on the CPU, in a temporary directory) and check that some pin catches each."""
import os
import subprocess

import pytest

import oracle
import pins

SRC = os.path.join(os.path.dirname(oracle.__file__), 'gdn2_oracle.c')

# (name, original text, planted text), or (name, [(original, planted), ...], None)
MUTANTS = [
    ('erase sign', 'e[j] = w[j] * v[j] - e[j];', 'e[j] = w[j] * v[j] + e[j];'),
    ('erase gate dropped', 'const double bk = b[c] * k[c];', 'const double bk = k[c];'),
    ('write gate dropped', 'e[j] = w[j] * v[j] - e[j];', 'e[j] = v[j] - e[j];'),
    ('decay dropped', 'const double a = exp(la[c]);', 'const double a = 1.0;'),
    ('decay sign', 'const double a = exp(la[c]);', 'const double a = exp(-la[c]);'),
    ('write uses q', 'S[(size_t)c * dv + j] += k[c] * e[j];', 'S[(size_t)c * dv + j] += q[c] * e[j];'),
    ('readout uses k', 'o[j] += S[(size_t)c * dv + j] * q[c];', 'o[j] += S[(size_t)c * dv + j] * k[c];'),
    # (I - (b*k) k^T) instead of (I - k (b*k)^T): e = S~^T k, S += k (w*v)^T - (b*k) e^T
    ('erase transposed', [('const double bk = b[c] * k[c];', 'const double bk = k[c];'),
                          ('S[(size_t)c * dv + j] += k[c] * e[j];',
                           'S[(size_t)c * dv + j] += k[c] * (w[j] * v[j]) - b[c] * k[c] * (w[j] * v[j] - e[j]);')], None),
    ('write gate on erase', 'const double bk = b[c] * k[c];', 'const double bk = w[c % dv] * k[c];'),
    ('state not carried', 'memcpy(S, J->S0 + sofs, sizeof(double) * (size_t)dk * dv);',
     'memset(S, 0, sizeof(double) * (size_t)dk * dv);'),
]


def _build(tmp_path, name, old, new):
    mut = open(SRC).read()
    edits = old if new is None else [(old, new)]
    for a, b in edits:
        assert a in mut, name
        mut = mut.replace(a, b, 1)
    c = tmp_path / 'm.c'
    c.write_text(mut)
    so = tmp_path / 'libm.so'
    subprocess.check_call(['gcc', '-O2', '-std=c11', '-fPIC', '-shared', '-pthread', '-o', str(so), str(c), '-lm'])
    return str(so)


@pytest.mark.parametrize('name,old,new', MUTANTS, ids=[m[0] for m in MUTANTS])
def test_some_pin_catches(tmp_path, name, old, new):
    lib = _build(tmp_path, name, old, new)

    def fwd(q, k, v, la, b, w, S0=None, cu_seqlens=None, B=None):
        return oracle.forward(q, k, v, la, b, w, S0, cu_seqlens=cu_seqlens, B=B, lib=lib)

    caught = []
    for pin in pins.ALL:
        try:
            pin(fwd)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f'no pin catches the planted mistake "{name}"'


# ---- the prologue oracle (numpy): planted mistakes in a copy of its source
import importlib.util

import oracle.prologue
import prologue_pins

PRO_SRC = oracle.prologue.__file__

PRO_MUTANTS = [
    ('conv taps reversed', 'acc += wt[:, :, j] * ext[t + j]', 'acc += wt[:, :, KERNEL - 1 - j] * ext[t + j]'),
    ('conv bias dropped', 'acc = bs.copy()', 'acc = np.zeros_like(bs)'),
    ('conv history ignored', 'before = np.transpose(np.asarray(history, dtype=np.float64)[i], (1, 0, 2))',
     'before = np.zeros((HIST, H, d))'),
    ('history taken from the start', 'hist_out[i] = np.transpose(ext[-HIST:], (1, 0, 2))',
     'hist_out[i] = np.transpose(ext[:HIST], (1, 0, 2))'),
    ('norm over the token axis', 'n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))',
     'n = np.sqrt(np.sum(x * x, axis=0, keepdims=True))'),
    ('norm not square-rooted', 'n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))',
     'n = np.sum(x * x, axis=-1, keepdims=True)'),
    ('sigmoid of -x', 'np.where(x >= 0, 1.0 / (1.0 + e), e / (1.0 + e))',
     'np.where(x >= 0, e / (1.0 + e), 1.0 / (1.0 + e))'),
    ('v normalised too', "return q, k, out['v'], sigmoid(b_logit)", "return q, k, l2_normalize(out['v']), sigmoid(b_logit)"),
    ('k left unnormalised', "k = l2_normalize(out['k'])", "k = out['k']"),
]


@pytest.mark.parametrize('name,old,new', PRO_MUTANTS, ids=[m[0] for m in PRO_MUTANTS])
def test_some_prologue_pin_catches(tmp_path, name, old, new):
    src = open(PRO_SRC).read()
    assert old in src, name
    path = tmp_path / 'prologue_mutant.py'
    path.write_text(src.replace(old, new, 1))
    spec = importlib.util.spec_from_file_location('oracle.prologue_mutant', str(path))
    mod = importlib.util.module_from_spec(spec)
    mod.__package__ = 'oracle'
    spec.loader.exec_module(mod)
    caught = []
    for pin in prologue_pins.ALL:
        try:
            pin(mod)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f'no pin catches the planted mistake "{name}"'


# ---- the gradient oracle (C): planted mistakes in a copy of its source
import backward_pins

BWD_SRC = os.path.join(os.path.dirname(oracle.__file__), 'gdn2_oracle_bwd.c')

BWD_MUTANTS = [
    ('dq from the previous state', 's += Snew[(size_t)c * dv + j] * dO[j];', 's += Sprev[(size_t)c * dv + j] * dO[j];'),
    ('readout gradient dropped', 'G[(size_t)c * dv + j] += q[c] * dO[j];', 'G[(size_t)c * dv + j] += 0.0 * q[c] * dO[j];'),
    ('erase term sign', 'dSd[(size_t)c * dv + j] = G[(size_t)c * dv + j] - b[c] * k[c] * dd[j];',
     'dSd[(size_t)c * dv + j] = G[(size_t)c * dv + j] + b[c] * k[c] * dd[j];'),
    ('erase-key gradient sign', 's -= Sd[(size_t)c * dv + j] * dd[j];', 's += Sd[(size_t)c * dv + j] * dd[j];'),
    ('decay gradient from the undecayed state', 's += dSd[(size_t)c * dv + j] * Sd[(size_t)c * dv + j];',
     's += dSd[(size_t)c * dv + j] * Sprev[(size_t)c * dv + j];'),
    ('state gradient not decayed', 'G[(size_t)c * dv + j] = al * dSd[(size_t)c * dv + j];',
     'G[(size_t)c * dv + j] = dSd[(size_t)c * dv + j];'),
    ('key gradient misses the erase path', 'dkk[c] += dbk[c] * b[c];', 'dkk[c] += 0.0 * dbk[c];'),
    ('write and value gradients swapped', [('dw[j] = dd[j] * v[j];', 'dw[j] = dd[j] * w[j];'),
                                           ('dvv[j] = dd[j] * w[j];', 'dvv[j] = dd[j] * v[j];')], None),
]


@pytest.mark.parametrize('name,old,new', BWD_MUTANTS, ids=[m[0] for m in BWD_MUTANTS])
def test_some_backward_pin_catches(tmp_path, name, old, new):
    mut = open(BWD_SRC).read()
    for a, b in (old if new is None else [(old, new)]):
        assert a in mut, name
        mut = mut.replace(a, b, 1)
    c = tmp_path / 'mb.c'
    c.write_text(mut)
    so = tmp_path / 'libmb.so'
    subprocess.check_call(['gcc', '-O2', '-std=c11', '-fPIC', '-shared', '-pthread', '-o', str(so), str(c), '-lm'])

    def bwd(*a, **kw):
        return oracle.backward(*a, **kw, lib=str(so))

    caught = []
    for pin in backward_pins.ALL:
        try:
            pin(bwd)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f'no pin catches the planted mistake "{name}"'
