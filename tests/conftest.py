import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def gpu_available():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def gdn():
    """The HIP library binding; GPU tests fail (not skip) if it cannot load."""
    import chunked_gated_delta_prefill_amd as lib
    lib.load()
    return lib


def pytest_terminal_summary(terminalreporter):
    """Every oracle comparison of the session, with its max normalised errors."""
    mod = sys.modules.get("_harness")
    recs = getattr(mod, "RECORDS", None)
    if not recs:
        return
    tr = terminalreporter
    tr.section("parity against the oracle (max normalised error)")
    worst = 0.0
    for label, eo, es, tol in recs:
        st = "-" if es is None else f"{es:.2e}"
        tr.write_line(f"{label:<58} out {eo:.2e}  state {st:>8}  tol {tol:g}")
        worst = max(worst, eo / tol, (es or 0.0) / tol)
    tr.write_line(f"{len(recs)} comparisons; worst error / tolerance = {worst:.3f}")
