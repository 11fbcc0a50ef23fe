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
