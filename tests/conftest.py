import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")


@pytest.fixture(scope="session")
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    return torch.device("cuda:0")


def pytest_terminal_summary(terminalreporter):
    """Parity margins of the run: each full-size workload on its own line,
    the element-wise cases as the worst one per dtype pair."""
    try:
        from parity import RESULTS
    except ImportError:
        return
    if not RESULTS:
        return
    import synth
    full = set(synth.CONFIGS) | set(synth.EXTRA_CONFIGS)
    w = terminalreporter.write_line
    w("parity: max|err|/RMS against the unrounded fp64 oracle (bound; * = not graded, bf16 output)")
    worst = {}
    for case, err, tol, graded, dts in RESULTS:
        if case in full:
            w(f"  {case:32s} {err:.3e}  ({tol:g}){'' if graded else ' *'}")
        else:
            key = (dts, graded)
            if key not in worst or err / tol > worst[key][1] / worst[key][2]:
                worst[key] = (case, err, tol, worst.get(key, (0, 0, 0, 0))[3] + 1)
            else:
                worst[key] = worst[key][:3] + (worst[key][3] + 1,)
    for (dts, graded), (case, err, tol, n) in sorted(worst.items()):
        w(f"  worst of {n:3d} {dts:11s} {err:.3e}  ({tol:g}){'' if graded else ' *'}  [{case}]")
