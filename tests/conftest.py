import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; runs the HIP library")
    config.addinivalue_line("markers", "slow: long-running case")


@pytest.fixture(scope="session")
def gpu():
    """The GPU device; GPU tests fail loudly (not skip) when none is present."""
    import torch
    assert torch.cuda.is_available(), "GPU test collected on a machine without a GPU"
    return torch.device("cuda:0")


def pytest_sessionfinish(session, exitstatus):
    """With QSA_STATS_OUT set, write the plain relative errors the score
    checks recorded (qsa_testlib.SCORE_STATS) to that file as JSON lines."""
    path = os.environ.get("QSA_STATS_OUT")
    if not path:
        return
    import json
    lib = sys.modules.get("qsa_testlib")
    if lib is None:
        return
    with open(path, "w") as f:
        for what, n, rel_max, share, zero_ref_nonzero in lib.SCORE_STATS:
            f.write(json.dumps({"what": what, "scores": n, "max_rel_err": rel_max, "share_within_1e-5": share,
                                "nonzero_where_ref_is_zero": zero_ref_nonzero}) + "\n")
