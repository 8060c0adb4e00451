"""Build libmoe.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Usage: python mixture_experts_layer_20_amd/build.py [-v]   (run by path: importing the
package loads the library this script builds)
Objects go to _build/ at the repository root; the library lands next to
this file.  Always recompiles every source.
"""
import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, 'csrc')
OUT = os.path.join(PKG, 'libmoe.so')
BUILD = os.path.join(ROOT, '_build')
ARCH = os.environ.get('MOE_OFFLOAD_ARCH', 'gfx950')

FLAGS = [
    '-O3', '-std=c++17', '-fPIC', f'--offload-arch={ARCH}',
    '-mcode-object-version=5',
    # packed float32 instructions stay off (written by neither hand nor compiler)
    '-Xclang', '-target-feature', '-Xclang', '-packed-fp32-ops',
    '-fvisibility=hidden', '-Wall', '-Wno-unused-function',
    '-I', os.path.join(ROOT, 'include'),
]


def hipcc():
    for c in (os.environ.get('HIPCC'), shutil.which('hipcc'), '/opt/rocm/bin/hipcc'):
        if c and os.path.exists(c):
            return c
    raise RuntimeError('hipcc not found')


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith('.hip'))


def _compile(src, verbose):
    obj = os.path.join(BUILD, os.path.basename(src) + '.o')
    cmd = [hipcc(), *FLAGS, '-c', src, '-o', obj]
    if verbose:
        print(' '.join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature for this target"
    err = '\n'.join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f'hipcc failed on {src}:\n{err}')
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    return obj


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with concurrent.futures.ThreadPoolExecutor(min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = OUT + '.tmp'
    cmd = [hipcc(), f'--offload-arch={ARCH}', '-shared', '-fPIC', *objs, '-o', tmp]
    if verbose:
        print(' '.join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError('link failed:\n' + r.stderr)
    os.replace(tmp, OUT)
    build_examples(verbose)
    return OUT


EXAMPLE = os.path.join(PKG, 'examples', 'forward_from_c.c')


def build_examples(verbose=False):
    """The plain-C consumer of the ABI (examples/forward_from_c.c), as a
    shared object for the tests and as a program, linked against libmoe.so
    and the HIP runtime only."""
    rocm = os.environ.get('ROCM_PATH', '/opt/rocm')
    base = ['gcc', '-std=c11', '-O2', '-Wall', '-D__HIP_PLATFORM_AMD__', '-I', os.path.join(rocm, 'include'),
            '-I', os.path.join(ROOT, 'include'), EXAMPLE, '-L', PKG, '-lmoe', '-L', os.path.join(rocm, 'lib'),
            '-lamdhip64', '-Wl,-rpath,$ORIGIN/..', '-Wl,-rpath,' + os.path.join(rocm, 'lib')]
    outdir = os.path.dirname(EXAMPLE)
    for extra, name in ((['-fPIC', '-shared'], 'libforward_from_c.so'), (['-DMOE_EXAMPLE_MAIN'], 'forward_from_c')):
        cmd = base[:1] + extra + base[1:] + ['-o', os.path.join(outdir, name)]
        if verbose:
            print(' '.join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f'building {name} failed:\n{r.stderr}')


if __name__ == '__main__':
    print(build(verbose='-v' in sys.argv))
