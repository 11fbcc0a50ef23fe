"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* The fp64 oracle (forward, decode, gradients) built with gcc and run on
  small packed batches by tests/sanitize/oracle_driver.c.
* The C ABI's host-side argument validation: every translation unit of
  libgdn2 with its host code built under the sanitizers, linked with
  tests/sanitize/abi_validation.c, which checks the status of each refused
  call (none launches a kernel).
"""
import concurrent.futures
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SAN = os.path.join(HERE, 'sanitize')
CSRC = os.path.join(ROOT, 'gated_delta_rule_wy_amd', 'csrc')
HIPCC = '/opt/rocm/bin/hipcc'
CLANGXX = '/opt/rocm/llvm/bin/clang++'
CLANG = '/opt/rocm/llvm/bin/clang'
ENV = dict(os.environ, ASAN_OPTIONS='detect_leaks=0:abort_on_error=1',
           UBSAN_OPTIONS='print_stacktrace=1:halt_on_error=1')


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f'{" ".join(cmd)} failed ({r.returncode}):\n{r.stdout}\n{r.stderr}'
    return r


def _check_clean(r):
    out = r.stdout + r.stderr
    assert 'runtime error' not in out and 'AddressSanitizer' not in out, out


@pytest.mark.skipif(shutil.which('gcc') is None, reason='gcc missing')
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / 'oracle_asan')
    _run(['gcc', '-O1', '-g', '-std=c11', '-pthread', '-fno-omit-frame-pointer',
          '-fsanitize=address,undefined', '-fno-sanitize-recover=undefined', '-o', exe,
          os.path.join(SAN, 'oracle_driver.c'), os.path.join(ROOT, 'oracle', 'gdn2_oracle.c'),
          os.path.join(ROOT, 'oracle', 'gdn2_oracle_bwd.c'), '-lm'])
    r = _run([exe], env=ENV, timeout=120)
    _check_clean(r)
    assert 'oracle driver: ok' in r.stdout


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANGXX)), reason='ROCm toolchain missing')
def test_abi_validation_under_sanitizers(tmp_path):
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith('.hip'))
    # the sanitizer flags apply to the host compilation only; the device code
    # is built as usual (and never launched: every call is refused first)
    flags = ['--offload-arch=gfx950', '-O1', '-g', '-std=c++17', '-fPIC', '-fno-omit-frame-pointer',
             '-Xclang', '-target-feature', '-Xclang', '-packed-fp32-ops',
             '-Xarch_host', '-fsanitize=address', '-Xarch_host', '-fsanitize=undefined']

    def compile_one(s):
        obj = str(tmp_path / (s[:-4] + '.o'))
        _run([HIPCC, *flags, '-c', '-o', obj, os.path.join(CSRC, s)])
        return obj

    with concurrent.futures.ThreadPoolExecutor(min(16, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, srcs))
    drv = str(tmp_path / 'abi_validation.o')
    _run([CLANG, '-O1', '-g', '-std=c11', '-fsanitize=address,undefined', '-c', '-o', drv,
          os.path.join(SAN, 'abi_validation.c')])
    exe = str(tmp_path / 'abi_asan')
    _run([CLANGXX, '-fsanitize=address,undefined', '-o', exe, drv, *objs, '-L/opt/rocm/lib', '-lamdhip64',
          '-Wl,-rpath,/opt/rocm/lib'])
    r = _run([exe], env=ENV, timeout=120)
    _check_clean(r)
    assert 'all expectations met' in r.stdout
