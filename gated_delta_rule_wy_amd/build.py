"""Build libgdn2.so in-tree with hipcc for gfx950 (no torch involved).

Every translation unit under csrc/ is compiled to an object file of its own,
several at once, and the objects are linked into one shared library.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, 'csrc')
OUT = os.path.join(HERE, 'libgdn2.so')

HIPCC = os.environ.get('HIPCC', '/opt/rocm/bin/hipcc')
FLAGS = ['-O3', '--offload-arch=gfx950', '-std=c++17', '-fPIC',
         # keep the compiler away from packed fp32 instructions
         '-Xclang', '-target-feature', '-Xclang', '-packed-fp32-ops']


def sources() -> list[str]:
    return sorted(f for f in os.listdir(CSRC) if f.endswith('.hip'))


def _jobs() -> int:
    env = os.environ.get('MAX_JOBS')
    n = int(env) if env and env.isdigit() else (os.cpu_count() or 1)
    return max(1, min(n, 16))


def _clean(stderr: str) -> str:
    return '\n'.join(l for l in stderr.splitlines() if 'packed-fp32-ops' not in l)


def build(verbose: bool = False) -> str:
    objdir = tempfile.mkdtemp(prefix='gdn2_build_')
    try:
        pending = list(sources())
        running: list[tuple[str, subprocess.Popen]] = []
        objs = []
        errors = []
        while pending or running:
            while pending and len(running) < _jobs():
                s = pending.pop(0)
                obj = os.path.join(objdir, s[:-4] + '.o')
                objs.append(obj)
                cmd = [HIPCC, *FLAGS, '-c', '-o', obj, os.path.join(CSRC, s)]
                if verbose:
                    print(' '.join(cmd), flush=True)
                running.append((s, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
            s, proc = running.pop(0)
            _, err = proc.communicate()
            if proc.returncode != 0:
                errors.append(f'hipcc failed on {s} ({proc.returncode}):\n{_clean(err)}')
            elif verbose and _clean(err).strip():
                print(_clean(err), file=sys.stderr)
        if errors:
            raise RuntimeError('\n'.join(errors))
        tmp = OUT + '.tmp'
        cmd = [HIPCC, '--offload-arch=gfx950', '-shared', '-fPIC', '-o', tmp, *objs]
        if verbose:
            print(' '.join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f'link failed ({res.returncode}):\n{_clean(res.stderr)}')
        os.replace(tmp, OUT)
    finally:
        shutil.rmtree(objdir, ignore_errors=True)
    return OUT


if __name__ == '__main__':
    print(build(verbose=True))
