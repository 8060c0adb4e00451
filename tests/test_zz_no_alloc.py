"""The dispatch entry point that allocates nothing (moe_dispatch_noalloc),
against moe_dispatch with a caller workspace, through the C ABI on an MI355X.

Two calls in a row, the second on a smaller batch, so that the second runs on
the scratch the first left behind; each result must equal moe_dispatch's bit
for bit (slots, drops, counts, the kept slots' tokens and the copied rows).
"""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu
DEV = 'cuda'


@pytest.fixture(scope='module')
def moe():
    assert torch.cuda.is_available(), 'GPU tests need a GPU'
    import mixture_experts_layer_20_amd as m
    return m


def _bufs(cfg, T, E, k, C, d, dropless):
    rows = T * k if dropless else E * C
    return dict(slot=torch.full((T, k), -7, dtype=torch.int32, device=DEV),
                dropped=torch.full((T, k), 9, dtype=torch.uint8, device=DEV),
                counts=torch.full((E,), -7, dtype=torch.int32, device=DEV),
                row_token=torch.full((max(rows, 1),), -7, dtype=torch.int32, device=DEV),
                xe=torch.zeros((max(rows, 1), d), dtype=torch.bfloat16, device=DEV))


def _one(moe, T, d, E, k, seed, **kw):
    print(f'noalloc dispatch T={T} d={d} E={E} k={k} {kw}', flush=True)
    cfg = moe.make_config(T, d, E, k, 64, capacity_factor=1.25, dtype='bf16', **kw)
    C = moe.moe_validate(cfg)
    idx = torch.from_numpy(synth.random_indices(T, E, k, seed=seed, skew=0.05)).to(DEV)
    x = torch.randn(T, d, device=DEV).to(torch.bfloat16)
    dl = bool(kw.get('dropless', False))
    ref = _bufs(cfg, T, E, k, C, d, dl)
    got = _bufs(cfg, T, E, k, C, d, dl)
    ws = moe.workspace(cfg, DEV)
    moe.moe_dispatch(cfg, x, idx, ref['slot'], ref['dropped'], ref['counts'], ref['row_token'], ref['xe'], ws)
    moe.moe_dispatch_noalloc(cfg, x, idx, got['slot'], got['dropped'], got['counts'], got['row_token'], got['xe'])
    torch.cuda.synchronize()
    for name in ('slot', 'dropped', 'counts'):
        assert torch.equal(got[name], ref[name]), name
    # the kept slots' tokens and rows (rows past an expert's kept count are untouched by both)
    assert torch.equal(got['row_token'], ref['row_token'])
    assert torch.equal(got['xe'].view(torch.int16), ref['xe'].view(torch.int16))
    assert int((ref['dropped'] == 0).sum()) > 0


@pytest.mark.parametrize('second', [dict(), dict(priority='token'), dict(dropless=True)])
def test_noalloc_dispatch_matches_the_workspace_entry_point(moe, second):
    # a large batch first (many histogram tiles), then a smaller one on the same scratch
    _one(moe, 9000, 256, 64, 6, seed=5)
    _one(moe, 300, 128, 8, 2, seed=6, **second)


def test_noalloc_dispatch_at_the_largest_stress_shape(moe):
    # 65,536 tokens, 128 experts, k = 8: 4 MiB of histograms
    _one(moe, 65536, 64, 128, 8, seed=7)
    _one(moe, 1, 64, 4, 2, seed=8)
