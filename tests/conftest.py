import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size case (minutes of CPU oracle work)")


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP library binding; skips when no GPU is visible, fails when the library is missing."""
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from hash_hierarchical_top_amd import hhr

    hhr.load()  # raises if libhhr.so is missing: no silent fallback
    return hhr


def pytest_sessionfinish(session, exitstatus):
    """Writes the excused-mismatch counts the GPU parity tests recorded (code bits, pages,
    blocks and tokens whose difference from the oracle lies inside the rounding band) to
    $HHR_EXCUSED_JSON, default gpurun_out/excused_mismatches.json."""
    gu = sys.modules.get("tests.gpu_util")
    if gu is None or not gu.EXCUSED:
        return
    import json

    path = os.environ.get("HHR_EXCUSED_JSON",
                          os.path.join(ROOT, "gpurun_out", "excused_mismatches.json"))
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w") as f:
        json.dump(gu.EXCUSED, f, indent=1, sort_keys=True)
