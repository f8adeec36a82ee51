import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def hbl():
    """The HIP library binding; GPU tests fail loudly if it is not built."""
    if not gpu_available():
        pytest.skip("no GPU visible")
    import bit_quantization_amd as hbl_pkg
    return hbl_pkg


def pytest_sessionfinish(session, exitstatus):
    """With HBL_PARITY_REPORT set to a path, write the worst parity figures
    met by the GPU tests of this session (tolerances are in parity_util)."""
    path = os.environ.get("HBL_PARITY_REPORT")
    if not path or "parity_util" not in sys.modules:
        return
    import json
    import parity_util
    with open(path, "w") as fh:
        json.dump(dict(parity_util.WORST, tolerances={"hadamard_rel": parity_util.HAD_TOL,
                                                      "scale_rel": parity_util.SCALE_TOL,
                                                      "output_rel_l2": parity_util.OUT_TOL,
                                                      "code_fraction": parity_util.CODE_FRAC}), fh, indent=1)
