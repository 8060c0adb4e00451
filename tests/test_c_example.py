"""The plain-C consumer of the ABI (mixture_experts_layer_20_amd/examples/
forward_from_c.c): it links against libmoe.so and the HIP runtime only, and
on a GPU its moe_forward matches the oracle."""
import ctypes
import os
import struct
import subprocess

import numpy as np
import pytest

import synth
from oracle import moe as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EX = os.path.join(ROOT, 'mixture_experts_layer_20_amd', 'examples')
LIB = os.path.join(EX, 'libforward_from_c.so')
PROG = os.path.join(EX, 'forward_from_c')


def test_example_links_only_the_library_and_the_hip_runtime():
    for path in (LIB, PROG):
        assert os.path.exists(path), f'{path} is not built: run mixture_experts_layer_20_amd/build.py'
        deps = subprocess.run(['ldd', path], capture_output=True, text=True, check=True).stdout
        names = {line.split()[0] for line in deps.splitlines() if '=>' in line}
        assert 'libmoe.so' in names and any(n.startswith('libamdhip64') for n in names)
        assert not any('torch' in n or 'python' in n for n in names), names


CASES = [synth.WORKLOADS['tiny_f32'],
         synth.Workload('cx', T=300, d=64, E=6, k=2, d_ff=128, act='gelu', score='softmax', renormalize=-1,
                        cf=1.0, dtype='f32', seed=81)]


@pytest.mark.gpu
@pytest.mark.parametrize('w', CASES, ids=[w.name for w in CASES])
def test_forward_from_plain_c_matches_the_oracle(tmp_path, w):
    inp = synth.router_inputs(w)
    ex = synth.all_expert_weights(w)
    src, dst = tmp_path / 'layer.bin', tmp_path / 'out.bin'
    with open(src, 'wb') as f:
        f.write(struct.pack('<5qd', w.T, w.d, w.E, w.k, w.d_ff, w.cf))
        for arr in (inp['x'], inp['w_router'], ex['w_in'], ex['b_in'], ex['w_out'], ex['b_out']):
            f.write(np.ascontiguousarray(synth.as_f32(arr), np.float32).tobytes())
    lib = ctypes.CDLL(LIB)
    lib.run_forward_case.restype = ctypes.c_int
    lib.run_forward_case.argtypes = [ctypes.c_char_p, ctypes.c_char_p]
    assert lib.run_forward_case(str(src).encode(), str(dst).encode()) == 0
    T, k, E, d = w.T, w.k, w.E, w.d
    raw = open(dst, 'rb').read()
    off = 0

    def take(dtype, n):
        nonlocal off
        a = np.frombuffer(raw, dtype, n, off)
        off += a.nbytes
        return a
    idx = take(np.int32, T * k).reshape(T, k)
    gates = take(np.float32, T * k).reshape(T, k)
    slot = take(np.int32, T * k).reshape(T, k)
    dropped = take(np.uint8, T * k).reshape(T, k).astype(bool)
    counts = take(np.int32, E)
    losses = take(np.float32, 2)
    stats = take(np.int32, 4)
    y = take(np.float32, T * d).reshape(T, d)
    assert off == len(raw)
    ref = O.moe_forward(w, inp, ex)
    np.testing.assert_array_equal(idx, ref['idx'])
    np.testing.assert_array_equal(slot, ref['slot'])
    np.testing.assert_array_equal(dropped, ref['dropped'])
    np.testing.assert_array_equal(counts, ref['counts'])
    assert stats.tolist() == [ref['stats'][kk] for kk in ('kept', 'dropped', 'fallback', 'pad')]
    assert np.abs(gates - ref['gates']).max() <= 1e-5 * np.abs(ref['gates']).max()
    assert np.abs(y - ref['y']).max() <= 1e-5 * np.abs(ref['y']).max()
    assert abs(losses[0] - ref['l_aux']) <= 1e-5 * abs(ref['l_aux'])
    assert abs(losses[1] - ref['l_z']) <= 1e-5 * abs(ref['l_z'])
