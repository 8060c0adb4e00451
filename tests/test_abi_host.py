"""Host-only checks of the C ABI: the library loads on a machine without a GPU,
exports every entry point include/moe.h declares, lays out its structs as the
header does, and validates configurations before touching the device."""
import ctypes
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, 'include', 'moe.h')
LIB = os.path.join(ROOT, 'mixture_experts_layer_20_amd', 'libmoe.so')


@pytest.fixture(scope='module')
def moe():
    if not os.path.exists(LIB):
        subprocess.run([sys.executable, os.path.join(ROOT, 'mixture_experts_layer_20_amd', 'build.py')],
                       check=True)
    import mixture_experts_layer_20_amd as m
    return m


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r'^MOE_API\s+(?:const\s+)?[a-z_0-9]+\*?\s+\*?(moe_[a-z_]+)\s*\(', text, re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ('moe_route', 'moe_dispatch', 'moe_expert_ffn', 'moe_combine', 'moe_forward',
              'moe_aux_losses', 'moe_validate', 'moe_workspace_bytes', 'moe_last_error',
              'moe_expert_ffn_packed', 'moe_expert_choice', 'moe_combine_expert_choice',
              'moe_dispatch_by_score', 'moe_backward', 'moe_backward_workspace_bytes'):
        assert n in names


def test_library_exports_every_declared_symbol(moe):
    out = subprocess.run(['nm', '-D', '--defined-only', moe.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r' T (\w+)$', out, re.M))
    for n in declared_functions():
        assert n in exported, n
    # nothing else of ours leaks out of the library
    ours = {s for s in exported if s.startswith('moe') or 'moe' in s.lower()}
    assert ours == set(declared_functions())
    lib = ctypes.CDLL(moe.LIB_PATH)
    for n in declared_functions():
        assert getattr(lib, n)


def test_one_hip_runtime_in_process(moe):
    maps = open('/proc/self/maps').read()
    libs = set(re.findall(r'(\S*libamdhip64\S*)', maps))
    assert len(libs) == 1, libs


def test_struct_layout_matches_header(tmp_path, moe):
    src = tmp_path / 'layout.c'
    src.write_text('''
#include <stdio.h>
#include <stddef.h>
#include "moe.h"
int main(void) {
  printf("%zu %zu %zu %zu %zu %zu %zu %zu %zu %zu %zu %zu\\n", sizeof(moe_config),
         offsetof(moe_config, capacity_factor), offsetof(moe_config, capacity_override),
         offsetof(moe_config, dropped_output), offsetof(moe_config, dropless), offsetof(moe_config, routing),
         offsetof(moe_config, save_preact), sizeof(moe_weights), sizeof(moe_outputs), offsetof(moe_outputs, lse),
         offsetof(moe_outputs, sel), sizeof(moe_grads));
  return 0;
}
''')
    exe = tmp_path / 'layout'
    subprocess.run(['gcc', '-std=c11', '-I', os.path.join(ROOT, 'include'), str(src), '-o', str(exe)],
                   check=True)
    got = list(map(int, subprocess.run([str(exe)], capture_output=True, text=True,
                                       check=True).stdout.split()))
    want = [ctypes.sizeof(moe.moe_config), moe.moe_config.capacity_factor.offset,
            moe.moe_config.capacity_override.offset, moe.moe_config.dropped_output.offset,
            moe.moe_config.dropless.offset, moe.moe_config.routing.offset, moe.moe_config.save_preact.offset,
            ctypes.sizeof(moe.moe_weights), ctypes.sizeof(moe.moe_outputs), moe.moe_outputs.lse.offset,
            moe.moe_outputs.sel.offset, ctypes.sizeof(moe.moe_grads)]
    assert got == want


def cfg(moe, **kw):
    base = dict(T=64, d=32, E=4, k=2, d_ff=64, capacity_factor=1.25, dtype='f32')
    base.update(kw)
    T, d, E, k, F = (base.pop(n) for n in ('T', 'd', 'E', 'k', 'd_ff'))
    return moe.make_config(T, d, E, k, F, **base)


def test_capacity_values(moe):
    assert moe.moe_validate(cfg(moe)) == 40
    assert moe.moe_validate(cfg(moe, T=4096, d=4096, E=8, k=2, d_ff=14336)) == 1280
    assert moe.moe_validate(cfg(moe, capacity_override=3)) == 3
    assert moe.moe_validate(cfg(moe, T=0)) == 0
    # every named workload
    sys.path.insert(0, ROOT)
    import synth
    from oracle import moe as O
    for w in synth.WORKLOADS.values():
        assert moe.moe_validate(moe.config_from_workload(w)) == O.capacity(w.T, w.k, w.E, w.cf)


@pytest.mark.parametrize('kw,msg', [
    (dict(capacity_factor=0.99), 'capacity_factor'),
    (dict(capacity_factor=float('nan')), 'capacity_factor'),
    # a capacity with no finite value, or one past the int64 range, is refused
    # before any integer conversion (it would otherwise wrap negative)
    (dict(capacity_factor=float('inf')), 'capacity_factor'),
    (dict(capacity_factor=1e300), 'capacity_factor'),
    (dict(capacity_factor=1e300, routing='expert'), 'capacity_factor'),
    (dict(capacity_factor=1e9), 'too large'),
    (dict(k=5), 'k must be'),
    (dict(k=0), 'k must be'),
    (dict(E=257, k=2), 'E must be'),
    (dict(E=64, k=33), 'k must be'),
    (dict(d=12), 'd must be'),
    (dict(d_ff=20), 'd_ff must be'),
    (dict(T=-1), 'T must be'),
    (dict(T=2 ** 29, k=4), 'T\\*k'),
    (dict(n_shared=1, d_ff_shared=0), 'd_ff_shared'),
    (dict(renormalize=2), 'renormalize'),
    (dict(score=7), 'score'),
    (dict(capacity_override=-1), 'capacity_override'),
])
def test_invalid_configs_raise(moe, kw, msg):
    with pytest.raises(ValueError, match=msg):
        moe.moe_validate(cfg(moe, **kw))
    assert moe.moe_workspace_bytes.__call__ is not None
    with pytest.raises(ValueError):
        moe.moe_workspace_bytes(cfg(moe, **kw))


def test_cf_below_one_is_fine_with_explicit_capacity(moe):
    assert moe.moe_validate(cfg(moe, capacity_factor=0.5, capacity_override=7)) == 7


def test_null_and_misaligned_pointers_rejected_before_launch(moe):
    lib = moe._lib
    c = cfg(moe)
    # moe_route with everything NULL: idx is required
    st = lib.moe_route(ctypes.byref(c), None, None, None, None, None, None, None, None, None, None,
                       None)
    assert st == moe.MOE_EINVAL and b'idx' in lib.moe_last_error()
    st = lib.moe_route(ctypes.byref(c), None, None, None, None, None, None, 16, 32, None, None, None)
    assert st == moe.MOE_EINVAL and b'logits' in lib.moe_last_error()
    st = lib.moe_route(ctypes.byref(c), 8, 64, None, None, None, None, 16, 32, None, None, None)
    assert st == moe.MOE_EINVAL and b'x must be 16-byte aligned' in lib.moe_last_error()
    bad = cfg(moe, capacity_factor=0.5)
    st = lib.moe_forward(ctypes.byref(bad), None, None, None, None, None)
    assert st == moe.MOE_EINVAL and b'capacity_factor' in lib.moe_last_error()
    st = lib.moe_forward(ctypes.byref(c), None, None, None, None, None)
    assert st == moe.MOE_EINVAL
    st = lib.moe_dispatch(ctypes.byref(c), None, 16, 16, 16, 16, None, None, None, None)
    assert st == moe.MOE_EINVAL and b'ws' in lib.moe_last_error()
    st = lib.moe_expert_ffn(ctypes.byref(c), 1, 4, 40, None, 16, None, 0, 16, None, None, 16, None, 12,
                            16, 16, None)
    assert st == moe.MOE_EINVAL and b'F must be' in lib.moe_last_error()
    st = lib.moe_expert_ffn(ctypes.byref(c), moe.MOE_SWIGLU, 4, 40, None, 16, None, 0, 16, 16, 16, 16,
                            None, 64, 16, 16, None)
    assert st == moe.MOE_EUNSUPPORTED
    st = lib.moe_expert_ffn(ctypes.byref(c), 1, 4, 40, None, 16, 16, 0, 16, None, None, 16, None, 64,
                            16, 16, None)
    assert st == moe.MOE_EINVAL and b'a_rows' in lib.moe_last_error()
    # biases, like every tensor, must be 16-byte aligned (the GEMM epilogue
    # reads four bf16 bias values per 8-byte load)
    for b_in, b_out, name in ((18, None, b'b_in'), (None, 24, b'b_out')):
        st = lib.moe_expert_ffn(ctypes.byref(c), 1, 4, 40, None, 16, None, 0, 16, None, b_in, 16, b_out,
                                64, 16, 16, None)
        assert st == moe.MOE_EINVAL and name + b' must be 16-byte aligned' in lib.moe_last_error()


def test_workspace_grows_with_capacity(moe):
    a = moe.moe_workspace_bytes(cfg(moe))
    b = moe.moe_workspace_bytes(cfg(moe, capacity_factor=4.0))
    assert 0 < a < b
    assert a % 256 == 0


def test_mixtral_workspace_is_its_expert_buffers_plus_a_few_mib(moe):
    """The forward workspace of the Mixtral-shaped layer: H [E*C, d_ff] and
    Ye [E*C, d] in bf16 (C = 2,560), the 64 MiB of float32 partial tiles of
    the tail split, and routing scratch of under 3 MiB; no dispatched copy
    of x."""
    import synth
    w = synth.WORKLOADS['mixtral_8x_top2']
    cfg = moe.config_from_workload(w)
    C = moe.moe_validate(cfg)
    assert C == 2560
    rows = w.E * C
    big = 2 * rows * w.d_ff + 2 * rows * w.d + (64 << 20)
    got = moe.moe_workspace_bytes(cfg)
    assert big <= got < big + (3 << 20)
    assert abs(got / 2**20 - 786.6) < 0.05


def test_dropless_capacity_and_workspace(moe):
    # dropless: C = T (a token picks an expert at most once), whatever the factor
    assert moe.moe_validate(cfg(moe, dropless=True)) == 64
    assert moe.moe_validate(cfg(moe, dropless=True, capacity_factor=0.5)) == 64
    assert moe.moe_validate(cfg(moe, dropless=True, capacity_override=3)) == 64
    c = cfg(moe, dropless=True)
    c.dropless = 2
    with pytest.raises(ValueError, match='dropless'):
        moe.moe_validate(c)
    # packed expert rows: T*k of them, not E*C; for the Mixtral shape the
    # dropless workspace is smaller than the capacity-factor-1.25 one
    big = dict(T=8192, d=4096, E=8, k=2, d_ff=14336, dtype='bf16', act='swiglu')
    assert moe.moe_workspace_bytes(cfg(moe, dropless=True, **big)) < moe.moe_workspace_bytes(cfg(moe, **big))


def test_packed_ffn_rejects_bad_arguments_before_launch(moe):
    lib = moe._lib
    c = cfg(moe)
    args = lambda groups, rows, total, F=64: (ctypes.byref(c), 0, groups, rows, total, 16, None, 0, 16, None, None,
                                              16, None, F, 16, 16, None)
    assert lib.moe_expert_ffn_packed(*args(257, 16, 100)) == moe.MOE_EINVAL
    assert b'groups' in lib.moe_last_error()
    assert lib.moe_expert_ffn_packed(*args(4, 16, -1)) == moe.MOE_EINVAL
    assert b'total_rows' in lib.moe_last_error()
    assert lib.moe_expert_ffn_packed(*args(4, None, 100)) == moe.MOE_EINVAL
    assert b'rows' in lib.moe_last_error()
    assert lib.moe_expert_ffn_packed(*args(4, 16, 100, F=12)) == moe.MOE_EINVAL
    # nothing to do: no launch, no pointer needed
    assert lib.moe_expert_ffn_packed(*args(4, None, 0)) == moe.MOE_OK


def test_balancing_entry_points_reject_bad_arguments(moe):
    lib = moe._lib
    c = cfg(moe)                                     # T = 64
    assert lib.moe_sequence_aux_loss(ctypes.byref(c), 48, 16, 16, 16, 256, None) == moe.MOE_EINVAL
    assert b'seq_len' in lib.moe_last_error()
    assert lib.moe_sequence_aux_loss(ctypes.byref(c), 0, 16, 16, 16, 256, None) == moe.MOE_EINVAL
    assert lib.moe_sequence_aux_loss(ctypes.byref(c), 16, None, 16, 16, 256, None) == moe.MOE_EINVAL
    assert b'probs' in lib.moe_last_error()
    assert lib.moe_update_select_bias(ctypes.byref(c), 16, 16, ctypes.c_float(-0.001), None) == moe.MOE_EINVAL
    assert b'gamma' in lib.moe_last_error()
    assert lib.moe_update_select_bias(ctypes.byref(c), None, 16, ctypes.c_float(0.001), None) == moe.MOE_EINVAL
    assert b'counts' in lib.moe_last_error()


def test_expert_choice_configuration(moe):
    # C from the same formula; the mode has no dropless variant; unknown modes fail
    assert moe.moe_validate(cfg(moe, routing='expert')) == 40
    assert moe.moe_validate(cfg(moe, routing='expert', capacity_override=100)) == 100
    with pytest.raises(ValueError, match='dropless'):
        moe.moe_validate(cfg(moe, routing='expert', dropless=True))
    c = cfg(moe)
    c.routing = 2
    with pytest.raises(ValueError, match='routing'):
        moe.moe_validate(c)
    # the transposed keys and the probabilities take workspace
    assert moe.moe_workspace_bytes(cfg(moe, routing='expert')) > moe.moe_workspace_bytes(cfg(moe))


def test_expert_choice_entry_points_reject_bad_arguments(moe):
    lib = moe._lib
    tc, ec = cfg(moe), cfg(moe, routing='expert')
    assert lib.moe_expert_choice(ctypes.byref(tc), 16, 16, 16, 16, 256, None) == moe.MOE_EINVAL
    assert b'MOE_EXPERT_CHOICE' in lib.moe_last_error()
    assert lib.moe_expert_choice(ctypes.byref(ec), None, 16, 16, 16, 256, None) == moe.MOE_EINVAL
    assert b'probs' in lib.moe_last_error()
    assert lib.moe_expert_choice(ctypes.byref(ec), 16, 16, None, 16, 256, None) == moe.MOE_EINVAL
    assert b'sel' in lib.moe_last_error()
    assert lib.moe_expert_choice(ctypes.byref(ec), 16, 16, 16, 16, None, None) == moe.MOE_EINVAL
    assert b'ws' in lib.moe_last_error()
    assert lib.moe_combine_expert_choice(ctypes.byref(tc), 16, 16, None, 16, 16, 16, None) == moe.MOE_EINVAL
    assert lib.moe_combine_expert_choice(ctypes.byref(ec), 16, 16, None, 16, 2, 16, None) == moe.MOE_EINVAL
    assert b'sel' in lib.moe_last_error()


def test_score_priority_configuration(moe):
    lib = moe._lib
    sc = cfg(moe, priority='score')
    assert moe.moe_validate(sc) == 40
    c = cfg(moe)
    c.priority = 3
    with pytest.raises(ValueError, match='priority'):
        moe.moe_validate(c)
    # the plain dispatch cannot rank by score; the score dispatch needs score priority
    assert lib.moe_dispatch(ctypes.byref(sc), None, 16, 16, 16, 16, None, None, 256, None) == moe.MOE_EINVAL
    assert b'moe_dispatch_by_score' in lib.moe_last_error()
    assert lib.moe_dispatch_by_score(ctypes.byref(cfg(moe)), None, 16, 16, 16, 16, 16, None, None, 256,
                                     None) == moe.MOE_EINVAL
    assert lib.moe_dispatch_by_score(ctypes.byref(sc), None, 16, None, 16, 16, 16, None, None, 256,
                                     None) == moe.MOE_EINVAL
    assert b'gates' in lib.moe_last_error()
    assert lib.moe_dispatch_by_score(ctypes.byref(sc), 16, 16, 16, 16, 16, 16, None, 16, 256,
                                     None) == moe.MOE_EINVAL
    assert b'row_token' in lib.moe_last_error()
    # its queue and the selection buffers take workspace
    assert moe.moe_workspace_bytes(sc) > moe.moe_workspace_bytes(cfg(moe))
    assert moe.moe_workspace_bytes(cfg(moe, priority='score', dropless=True)) == \
        moe.moe_workspace_bytes(cfg(moe, dropless=True))


def test_backward_configuration(moe):
    lib = moe._lib
    bf = dict(dtype='bf16')
    assert lib.moe_backward_workspace_bytes(ctypes.byref(cfg(moe, **bf))) > 0
    # built for bf16: token choice with a capacity or dropless, expert choice
    assert lib.moe_backward_workspace_bytes(ctypes.byref(cfg(moe))) == 0             # f32
    assert lib.moe_backward_workspace_bytes(ctypes.byref(cfg(moe, dropless=True, **bf))) > 0
    assert lib.moe_backward_workspace_bytes(ctypes.byref(cfg(moe, routing='expert', **bf))) > 0
    c = cfg(moe)
    g = moe.moe_grads()
    assert lib.moe_backward(ctypes.byref(c), None, None, None, None, None, 0.0, 0.0, ctypes.byref(g), None,
                            None) == moe.MOE_EUNSUPPORTED
    c = cfg(moe, **bf)
    assert lib.moe_backward(ctypes.byref(c), None, None, None, None, None, 0.0, 0.0, ctypes.byref(g), None,
                            None) == moe.MOE_EINVAL
    assert b'NULL' in lib.moe_last_error()


def test_save_preact_configuration(moe):
    bf = dict(dtype='bf16')
    assert moe.moe_validate(cfg(moe, save_preact=True, **bf)) == 40
    assert moe.moe_validate(cfg(moe, save_preact=True, dropless=True, **bf)) == 64
    assert moe.moe_validate(cfg(moe, save_preact=True, routing='expert', **bf)) > 0
    with pytest.raises(ValueError, match='save_preact'):
        moe.moe_validate(cfg(moe, save_preact=True))                                    # f32
    # the forward keeps them, the backward need not
    assert moe.moe_workspace_bytes(cfg(moe, save_preact=True, **bf)) > moe.moe_workspace_bytes(cfg(moe, **bf))
    assert moe.moe_backward_workspace_bytes(cfg(moe, save_preact=True, **bf)) < \
        moe.moe_backward_workspace_bytes(cfg(moe, **bf))


def test_backward_binding_checks_the_per_token_gradient_sizes(moe):
    """The gate gradients are [T,k] under token choice and [T,E] under expert
    choice; a buffer of the other size is refused before the library runs."""
    import torch
    for routing, bad in (('token', (64, 4)), ('expert', (64, 2))):
        c = cfg(moe, dtype='bf16', routing=routing)
        with pytest.raises(ValueError, match='dgates'):
            moe.moe_backward(c, {}, None, {}, None, None, {'dgates': torch.empty(*bad)}, None)
    with pytest.raises(ValueError, match='dlogits'):
        moe.moe_backward(cfg(moe, dtype='bf16'), {}, None, {}, None, None, {'dlogits': torch.empty(64, 2)}, None)


def test_noalloc_dispatch_rejects_oversized_configurations_before_launch(moe):
    # 200,000 tokens x k 8 x 256 experts need 25 MB of histograms: more than
    # the fixed 16 MiB scratch; refused on the host (no device is touched)
    c = cfg(moe, T=200000, E=256, k=8, d=64, dtype='bf16')
    lib = moe._lib
    fake = ctypes.c_void_p(1 << 20)
    st = lib.moe_dispatch_noalloc(ctypes.byref(c), None, fake, fake, fake, fake, None, None, None)
    assert st == moe.MOE_EINVAL
    msg = lib.moe_last_error()
    assert b'noalloc' in msg and b'scratch' in msg
    # invalid configurations are refused as by moe_dispatch
    bad = cfg(moe, capacity_factor=0.5)
    assert lib.moe_dispatch_noalloc(ctypes.byref(bad), None, fake, fake, fake, fake, None, None, None) == moe.MOE_EINVAL
