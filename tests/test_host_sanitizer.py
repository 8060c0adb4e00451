"""The library's host code (validation, capacity arithmetic, workspace
carving) built with AddressSanitizer and UndefinedBehaviorSanitizer (host
side only: -Xarch_host), linked into a plain-C driver that exercises those
paths without a GPU, and run on the CPU.  Any sanitizer report or failed
expectation fails the test."""
import concurrent.futures
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, 'mixture_experts_layer_20_amd', 'csrc')
SAN = ['-Xarch_host', '-fsanitize=address,undefined', '-Xarch_host', '-fno-sanitize-recover=all',
       '-Xarch_host', '-fno-omit-frame-pointer']


def hipcc():
    for c in (os.environ.get('HIPCC'), shutil.which('hipcc'), '/opt/rocm/bin/hipcc'):
        if c and os.path.exists(c):
            return c
    return None


@pytest.mark.slow
def test_host_code_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    cc = hipcc()
    if cc is None:
        pytest.skip('hipcc not available')
    flags = ['-O1', '-g', '-std=c++17', '-fPIC', '--offload-arch=gfx950', '-Xclang', '-target-feature',
             '-Xclang', '-packed-fp32-ops', '-I', os.path.join(ROOT, 'include')] + SAN

    def comp(src):
        obj = str(tmp_path / (os.path.basename(src) + '.o'))
        r = subprocess.run([cc, *flags, '-c', src, '-o', obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        return obj

    srcs = sorted(glob.glob(os.path.join(CSRC, '*.hip')))
    with concurrent.futures.ThreadPoolExecutor(min(8, len(srcs))) as ex:
        objs = list(ex.map(comp, srcs))
    drv = str(tmp_path / 'host_checks.o')
    r = subprocess.run([cc, '-x', 'c', '-O1', '-g', '-I', os.path.join(ROOT, 'include'), *SAN, '-c',
                        os.path.join(ROOT, 'tests', 'host', 'host_checks.c'), '-o', drv],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    exe = str(tmp_path / 'host_checks')
    r = subprocess.run([cc, '--offload-arch=gfx950', *SAN, drv, *objs, '-o', exe, '-lm'], capture_output=True,
                       text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS='detect_leaks=0:halt_on_error=1',
               UBSAN_OPTIONS='print_stacktrace=1:halt_on_error=1')
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert 'runtime error' not in out and 'AddressSanitizer' not in out, out[-4000:]
    assert 'host checks passed' in out
