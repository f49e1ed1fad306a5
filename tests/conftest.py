import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def rng():
    import numpy as np
    return np.random.default_rng(12345)


# routing-protocol records of the fused-layer parity tests (changed tokens, near ties, errors),
# printed at the end of the session so that they appear in the run's output
_ROUTING = []


def record_routing(name, rec):
    _ROUTING.append((name, rec))


def pytest_terminal_summary(terminalreporter):
    if not _ROUTING:
        return
    tr = terminalreporter
    tr.write_sep("-", "fused-layer routing against the oracle")
    for name, r in _ROUTING:
        tr.write_line(f"{name} T={r['T']}: changed {r['changed']}, near-ties {r['near_ties']}, "
                      f"min margin {r['min_margin']:.3g}, max logit err {r['max_logit_err']:.3g}, "
                      f"logits rel-L2 {r['logits_rel_l2']:.3g}, y rel-L2 {r['y_rel_l2']:.3g}, "
                      f"kept {r['kept']}, dropped {r['dropped']}")
