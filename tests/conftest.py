import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line('markers', 'gpu: needs an MI355X (gfx950) GPU and the built HIP library')
    config.addinivalue_line('markers', 'slow: takes more than a few seconds on the CPU')


def pytest_terminal_summary(terminalreporter):
    """The errors the GPU comparisons measured, one line per test: the worst
    max-relative error of each quantity (the bars: 1e-5 for float32 outputs
    and the losses, 2e-2 for bf16 outputs and gradients)."""
    helpers = sys.modules.get('gpu_helpers')
    if helpers is None or not helpers.PARITY:
        return
    tr = terminalreporter
    tr.section('measured parity errors (max-relative, worst per test)')
    for test, row in helpers.PARITY.items():
        tr.write_line(f'{test}  ' + '  '.join(f'{q} {e:.1e}' for q, e in row.items()))
