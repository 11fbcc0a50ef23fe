"""Build libgdn2.so in-tree with hipcc for gfx950 (no torch involved)."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, 'csrc')
SOURCES = ['api.hip', 'decode.hip', 'chunk.hip']
OUT = os.path.join(HERE, 'libgdn2.so')

HIPCC = os.environ.get('HIPCC', '/opt/rocm/bin/hipcc')
FLAGS = ['-O3', '--offload-arch=gfx950', '-std=c++17', '-fPIC', '-shared',
         # keep the compiler away from packed fp32 instructions
         '-Xclang', '-target-feature', '-Xclang', '-packed-fp32-ops']


def build(verbose: bool = False) -> str:
    tmp = OUT + '.tmp'
    cmd = [HIPCC, *FLAGS, '-o', tmp] + [os.path.join(CSRC, s) for s in SOURCES]
    if verbose:
        print(' '.join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = '\n'.join(l for l in res.stderr.splitlines() if 'packed-fp32-ops' not in l)
    if res.returncode != 0:
        raise RuntimeError(f'hipcc failed ({res.returncode}):\n{err}')
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, OUT)
    return OUT


if __name__ == '__main__':
    print(build(verbose=True))
